// C ABI of the QMoE library: host-side validation, workspace layout, variant choice
// from shapes only, and launches on the caller's stream. See include/qmoe.h.
#include "qmoe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_error;
// armed timing pairs, oldest first
constexpr int kTimingSlots = 4;
thread_local qmoe::GemmTiming g_timing[kTimingSlots];
thread_local int g_timing_n = 0;

qmoe_status fail(qmoe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

qmoe_status ok() {
  g_error.clear();
  return QMOE_OK;
}

qmoe_status device_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QMOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace qmoe {

qmoe_status fail_with(qmoe_status st, const char* msg, const char* detail) {
  return (detail && detail[0]) ? fail(st, "%s: %s", msg, detail) : fail(st, "%s", msg);
}

void set_gemm_timing(hipEvent_t start, hipEvent_t stop) {
  if (start == nullptr && stop == nullptr) {
    g_timing_n = 0;
    return;
  }
  if (g_timing_n < kTimingSlots) g_timing[g_timing_n++] = GemmTiming{start, stop};
}

GemmTiming take_gemm_timing() {
  if (g_timing_n == 0) return GemmTiming{};
  const GemmTiming t = g_timing[0];
  for (int i = 1; i < g_timing_n; ++i) g_timing[i - 1] = g_timing[i];
  --g_timing_n;
  return t;
}

}  // namespace qmoe

namespace {

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

constexpr int64_t kMaxExperts = 512;
constexpr int64_t kMaxTopK = 32;
constexpr int kMaxBlock = 512;
constexpr int64_t kF32LdsBytes = 48 * 1024;

bool swiglu(const qmoe_params* p) { return p->activation == QMOE_ACT_SWIGLU; }
bool has_fc3(const qmoe_params* p) { return swiglu(p) && p->swiglu_fusion == 0; }
int64_t n1_rows(const qmoe_params* p) {
  return (swiglu(p) && p->swiglu_fusion != 0) ? 2 * p->inter_size : p->inter_size;
}

// Rows per expert tile, from shapes only: 128-row MFMA tiles when an expert is expected
// to receive at least 64 rows (prefill) and the 128-row grid still has some 512 or more
// workgroups (a single expert, as in the linear layer, gives few tiles); 32-row
// weight-streaming tiles from 12 expected rows on, so that an expert's 17-32 rows read its
// weights once, not twice; 16-row tiles below.
int32_t default_tile_m(const qmoe_params* p) {
  if (p->act_dtype == QMOE_BF16) {
    const int64_t a = p->num_tokens * p->k;
    const int64_t tiles128 = std::max<int64_t>(a / 128, std::min(p->num_experts, a));
    const int64_t cols128 = std::min(p->hidden_size, p->inter_size) / 128;
    if (a >= 64 * p->num_experts && tiles128 * cols128 >= 512) return 128;
    return a >= 12 * p->num_experts ? 32 : 16;
  }
  const int64_t kmax = std::max(p->hidden_size, p->inter_size);
  int32_t m = 16;
  while (m > 1 && m * kmax * 4 > kF32LdsBytes) m >>= 1;
  return m;
}

int32_t tile_m_of(const qmoe_params* p) { return p->tile_m > 0 ? p->tile_m : default_tile_m(p); }

qmoe_status validate(const qmoe_params* p) {
  if (!p) return fail(QMOE_ERR_UNBOUND, "params is NULL");
  if (p->num_tokens < 0) return fail(QMOE_ERR_INVALID, "num_tokens %lld < 0", (long long)p->num_tokens);
  if (p->hidden_size < 1 || p->inter_size < 1)
    return fail(QMOE_ERR_INVALID, "hidden_size and inter_size must be positive");
  if (p->num_experts < 1 || p->num_experts > kMaxExperts)
    return fail(QMOE_ERR_UNSUPPORTED, "num_experts %lld outside [1, %lld]",
                (long long)p->num_experts, (long long)kMaxExperts);
  if (p->k < 1 || p->k > p->num_experts)
    return fail(QMOE_ERR_INVALID, "k %lld outside [1, num_experts]", (long long)p->k);
  if (p->k > kMaxTopK) return fail(QMOE_ERR_UNSUPPORTED, "k %lld > %lld", (long long)p->k, (long long)kMaxTopK);
  if (p->n_group > 1) {
    if (p->n_group > qmoe::kMaxGroups)
      return fail(QMOE_ERR_UNSUPPORTED, "n_group %d > %d", p->n_group, qmoe::kMaxGroups);
    if (p->num_experts % p->n_group)
      return fail(QMOE_ERR_INVALID, "num_experts %lld is not a multiple of n_group %d",
                  (long long)p->num_experts, p->n_group);
    if (p->topk_group < 1 || p->topk_group > p->n_group)
      return fail(QMOE_ERR_INVALID, "topk_group %d outside [1, n_group]", p->topk_group);
    if (p->k > p->topk_group * (p->num_experts / p->n_group))
      return fail(QMOE_ERR_INVALID, "k %lld exceeds the experts of topk_group groups",
                  (long long)p->k);
  } else if (p->n_group < 0 || p->topk_group < 0) {
    return fail(QMOE_ERR_INVALID, "n_group and topk_group must not be negative");
  }
  if (!std::isfinite(p->routed_scaling_factor))
    return fail(QMOE_ERR_INVALID, "routed_scaling_factor must be finite");
  if (p->compute_mode != QMOE_COMPUTE_FLOAT && p->compute_mode != QMOE_COMPUTE_INT8)
    return fail(QMOE_ERR_INVALID, "compute_mode %d unknown", p->compute_mode);
  if (p->compute_mode == QMOE_COMPUTE_INT8 && p->block_size == 0)
    return fail(QMOE_ERR_INVALID, "the int8 activation tier needs block_size > 0");
  // The tier decides the codes of h from h itself. An fp32 h that differs from an exact
  // evaluation in its last bit (summation order) can move a code by one step, and one step
  // is worth more than the fp32 path's error bound, so fp32 activations keep the float
  // path; the rounding itself (qmoe_quantize_act) serves both dtypes.
  if (p->compute_mode == QMOE_COMPUTE_INT8 && p->act_dtype == QMOE_F32)
    return fail(QMOE_ERR_UNSUPPORTED, "the int8 activation tier runs with bf16 activations");
  if (p->expert_weight_bits != 4 && p->expert_weight_bits != 8)
    return fail(QMOE_ERR_INVALID, "expert_weight_bits %d is not 4 or 8", p->expert_weight_bits);
  if (p->block_size != 0 && (!is_pow2(p->block_size) || p->block_size < 16))
    return fail(QMOE_ERR_INVALID, "block_size %d must be 0 or a power of two >= 16", p->block_size);
  if (p->block_size > kMaxBlock)
    return fail(QMOE_ERR_UNSUPPORTED, "block_size %d > %d", p->block_size, kMaxBlock);
  if (p->activation < QMOE_ACT_SWIGLU || p->activation > QMOE_ACT_GELU)
    return fail(QMOE_ERR_INVALID, "activation %d unknown", p->activation);
  if (p->activation == QMOE_ACT_GELU && p->gelu_mode != 0 && p->gelu_mode != 1)
    return fail(QMOE_ERR_INVALID, "gelu_mode %d is not 0 (erf) or 1 (tanh)", p->gelu_mode);
  if (!std::isfinite(p->expert_output_scale))
    return fail(QMOE_ERR_INVALID, "expert_output_scale must be finite");
  if (p->apply_router_weight_on_input && p->compute_mode == QMOE_COMPUTE_INT8)
    return fail(QMOE_ERR_UNSUPPORTED,
                "the int8 tier with the routing weight on the input (the codes would depend "
                "on each slot's weight)");
  if (p->use_sparse_mixer) {
    if (p->k != 2 || p->num_experts < 2)
      return fail(QMOE_ERR_INVALID, "the sparse mixer picks k = 2 experts (k %lld, E %lld)",
                  (long long)p->k, (long long)p->num_experts);
    if (p->normalize_routing_weights)
      return fail(QMOE_ERR_INVALID, "the sparse mixer's weights are not renormalised");
    if (p->n_group > 1 || p->e_score_correction_bias)
      return fail(QMOE_ERR_INVALID, "the sparse mixer takes no grouping and no selection bias");
    if (!std::isfinite(p->sparse_mixer_eps) || p->sparse_mixer_eps < 0.f)
      return fail(QMOE_ERR_INVALID, "sparse_mixer_eps must be finite and >= 0");
  }
  if (p->swiglu_fusion < 0 || p->swiglu_fusion > 2)
    return fail(QMOE_ERR_INVALID, "swiglu_fusion %d outside {0, 1, 2}", p->swiglu_fusion);
  if (!swiglu(p) && p->swiglu_fusion != 0)
    return fail(QMOE_ERR_INVALID, "swiglu_fusion must be 0 unless the activation is swiglu");
  if (p->act_dtype != QMOE_F32 && p->act_dtype != QMOE_BF16)
    return fail(QMOE_ERR_DTYPE, "act_dtype %d unknown", p->act_dtype);
  if (p->scale_dtype != QMOE_F32 && p->scale_dtype != QMOE_BF16 && p->scale_dtype != QMOE_E8M0)
    return fail(QMOE_ERR_DTYPE, "scale_dtype %d unknown", p->scale_dtype);
  if (p->scale_dtype == QMOE_E8M0) {
    // MX FP4: E2M1 codes, one E8M0 scale per 32 k
    if (p->expert_weight_bits != 4 || p->block_size != 32)
      return fail(QMOE_ERR_INVALID, "E8M0 scales (MX FP4) need expert_weight_bits 4 and block_size 32");
    if (p->act_dtype != QMOE_BF16 || p->weight_layout != QMOE_LAYOUT_TILES)
      return fail(QMOE_ERR_UNSUPPORTED,
                  "MX FP4 weights run with bf16 activations in the tiled layout (qmoe_pack_stack)");
  }
  if (p->weight_layout != QMOE_LAYOUT_ROWS && p->weight_layout != QMOE_LAYOUT_TILES)
    return fail(QMOE_ERR_INVALID, "weight_layout %d unknown", p->weight_layout);
  if (p->weight_layout == QMOE_LAYOUT_TILES && p->act_dtype != QMOE_BF16)
    return fail(QMOE_ERR_UNSUPPORTED, "the tiled weight layout serves bf16 activations only");
  const int pack = 8 / p->expert_weight_bits;
  if (p->hidden_size % pack || p->inter_size % pack)
    return fail(QMOE_ERR_SHAPE, "hidden_size and inter_size must be multiples of %d", pack);
  if (p->strict_blocks && p->block_size &&
      (p->hidden_size % p->block_size || p->inter_size % p->block_size))
    return fail(QMOE_ERR_SHAPE, "hidden_size and inter_size must be multiples of block_size %d",
                p->block_size);
  if (p->num_tokens * p->k >= (int64_t(1) << 31))
    return fail(QMOE_ERR_UNSUPPORTED, "num_tokens * k must stay below 2^31");
  const int32_t m = tile_m_of(p);
  if (p->act_dtype == QMOE_BF16) {
    if (p->hidden_size % 32 || p->inter_size % 32)
      return fail(QMOE_ERR_UNSUPPORTED, "bf16 path needs hidden_size and inter_size multiples of 32");
    if (m != 16 && m != 32 && m != 128)
      return fail(QMOE_ERR_UNSUPPORTED, "bf16 path needs tile_m 16, 32 or 128 (got %d)", m);
    // 32-bit buffer offsets: activations, h and one expert's stack must stay below 2 GiB
    const int64_t kmax = std::max(p->hidden_size, p->inter_size);
    const int64_t rows_max = ((p->num_tokens * p->k) / m + std::min<int64_t>(p->num_experts, p->num_tokens * p->k)) * m;
    if (p->num_tokens * p->hidden_size * 2 >= (int64_t(1) << 31) ||
        rows_max * p->inter_size * 2 >= (int64_t(1) << 31) ||
        2 * p->inter_size * kmax * p->expert_weight_bits / 8 >= (int64_t(1) << 31))
      return fail(QMOE_ERR_UNSUPPORTED, "bf16 path: a tensor or one expert's stack reaches 2 GiB");
    if (p->block_size) {
      const int64_t nb = (kmax + p->block_size - 1) / p->block_size;
      const int64_t sbytes = p->scale_dtype == QMOE_BF16 ? 2 : (p->scale_dtype == QMOE_E8M0 ? 1 : 4);
      if (2 * 64 * nb * sbytes > 64 * 1024)
        return fail(QMOE_ERR_UNSUPPORTED, "bf16 path: %lld scales per row do not fit in LDS",
                    (long long)nb);
    }
  } else {
    const int64_t kmax = std::max(p->hidden_size, p->inter_size);
    if (m < 1 || m > 16 || m * kmax * 4 > kF32LdsBytes)
      return fail(QMOE_ERR_UNSUPPORTED, "f32 path: tile_m %d with K %lld does not fit", m,
                  (long long)kmax);
  }
  return ok();
}

// The packing ignores weight_layout; MX FP4 parameters are checked as they will be used
// (tiled layout).
qmoe_status validate_for_pack(const qmoe_params* p) {
  if (p && p->scale_dtype == QMOE_E8M0) {
    qmoe_params q = *p;
    q.weight_layout = QMOE_LAYOUT_TILES;
    return validate(&q);
  }
  return validate(p);
}

qmoe::RouteOpts route_opts(const qmoe_params* p) {
  qmoe::RouteOpts o{};
  o.bias = p->e_score_correction_bias;
  o.n_group = p->n_group > 1 ? p->n_group : 1;
  o.topk_group = p->n_group > 1 ? p->topk_group : 1;
  o.scale = p->routed_scaling_factor != 0.f ? p->routed_scaling_factor : 1.f;
  o.mixer = p->use_sparse_mixer != 0;
  o.mixer_eps = p->sparse_mixer_eps;
  return o;
}

qmoe::CombineOpts combine_opts(const qmoe_params* p) {
  qmoe::CombineOpts c{};
  c.weights = p->apply_router_weight_on_input ? 0 : 1;
  c.scale = p->expert_output_scale != 0.f ? p->expert_output_scale : 1.f;
  return c;
}

int64_t max_tiles_of(const qmoe_params* p) {
  const int64_t A = p->num_tokens * p->k;
  const int32_t m = tile_m_of(p);
  return A / m + std::min<int64_t>(p->num_experts, A);
}

int64_t max_rows_of(const qmoe_params* p) { return max_tiles_of(p) * tile_m_of(p); }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// The int8 tier's dot on the int8 matrix cores: prefill-sized tiles of the tiled layout with
// integer codes, blocks of 64 and 128 (shorter blocks ran faster on the bf16 kernels), and
// both contraction lengths multiples of 64 (the codes' 64-groups); elsewhere the tier's
// rounded activations take the bf16 kernels.
bool use_i8_dot(const qmoe_params* p) {
  return p->compute_mode == QMOE_COMPUTE_INT8 && p->act_dtype == QMOE_BF16 &&
         p->weight_layout == QMOE_LAYOUT_TILES && p->scale_dtype != QMOE_E8M0 &&
         tile_m_of(p) == 128 && (p->block_size == 64 || p->block_size == 128) &&
         p->hidden_size % 64 == 0 && p->inter_size % 64 == 0;
}

// The forward forms each token's row sum once for fc1 (launch_rowsum): the 128-row
// per-row-scale kernel on tiled weights takes its zero-point correction from it.
bool use_xsum(const qmoe_params* p) {
  return p->compute_mode == QMOE_COMPUTE_FLOAT && p->act_dtype == QMOE_BF16 &&
         p->weight_layout == QMOE_LAYOUT_TILES && p->scale_dtype != QMOE_E8M0 &&
         p->block_size == 0 && tile_m_of(p) == 128;
}

// The fp16 block-scale path: 4-bit codes with bf16 block scales of 16 to 128 at 128-row
// tiles in the tiled layout, bf16 activations. The forward lifts x and h into fp16 and the
// weight rows' scales by powers of two (launch_prep_f16, launch_rows_to_f16), and the GEMMs
// take each weight exactly as one fp16 operand (gemm_prefill_h16_kernel.h). The stage entry
// points, which have no workspace for the fp16 rows, keep the bf16 kernels.
bool use_h16(const qmoe_params* p) {
  return p->compute_mode == QMOE_COMPUTE_FLOAT && p->act_dtype == QMOE_BF16 &&
         p->weight_layout == QMOE_LAYOUT_TILES && p->scale_dtype == QMOE_BF16 &&
         p->expert_weight_bits == 4 && p->block_size >= 16 && p->block_size <= 128 &&
         tile_m_of(p) == 128 && p->hidden_size % 8 == 0 && p->inter_size % 8 == 0;
}

// With 4-bit codes on that path fc1 also writes each row's partial sums of h, one per
// column block; launch_partsum adds them up, and fc2 takes its zero point's correction from
// those row sums.
bool use_hpart(const qmoe_params* p) { return use_xsum(p) && p->expert_weight_bits == 4; }
int hpart_blocks(const qmoe_params* p) {
  const int cols = qmoe::prefill_rows_fc1_cols(swiglu(p) ? qmoe::kModeSwiglu : qmoe::kModePlainAct);
  return static_cast<int>((p->inter_size + cols - 1) / cols);
}

struct Workspace {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_assign;
  int32_t* assign_pos;
  int32_t* tiles;
  int32_t* num_tiles;
  void* perm_scratch;
  void* h;
  float* y;
  void* xq;  // the int8-tier copy of x (compute_mode QMOE_COMPUTE_INT8)
  // the int8 dot (use_i8_dot): codes and block factors of x and of h
  int8_t* xc;
  float* xf;
  int8_t* hc;
  float* hf;
  float* xsum;  // use_xsum: the row sums of x
  float* hpart;  // use_hpart: fc1's partial row sums of h [qmoe_max_rows, hpart_blocks]
  float* hsum;   // use_hpart: the row sums of h [qmoe_max_rows]
  // use_h16: x and h as lifted fp16 rows with their lifts, and the lifts of the weight rows'
  // scales (fc1, fc3 when separate, fc2)
  void* x16;
  int32_t* xlift;
  void* h16;
  int32_t* hlift;
  int32_t* w1lift;
  int32_t* w3lift;
  int32_t* w2lift;
  size_t bytes;
};

Workspace carve(const qmoe_params* p, char* base) {
  const int64_t A = p->num_tokens * p->k;
  const int64_t rows = max_rows_of(p);
  const size_t act = p->act_dtype == QMOE_BF16 ? 2 : 4;
  Workspace w{};
  size_t off = 0;
  // with a null base the pieces' addresses are their byte offsets
  auto take = [&](size_t bytes) {
    char* ptr = reinterpret_cast<char*>(reinterpret_cast<uintptr_t>(base) + off);
    off += align256(bytes);
    return ptr;
  };
  w.topk_ids = reinterpret_cast<int32_t*>(take(A * 4));
  w.topk_w = reinterpret_cast<float*>(take(A * 4));
  w.counts = reinterpret_cast<int32_t*>(take(p->num_experts * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((p->num_experts + 1) * 4));
  w.sorted_assign = reinterpret_cast<int32_t*>(take(rows * 4));
  w.assign_pos = reinterpret_cast<int32_t*>(take(A * 4));
  w.tiles = reinterpret_cast<int32_t*>(take(max_tiles_of(p) * 8));
  w.num_tiles = reinterpret_cast<int32_t*>(take(4));
  w.perm_scratch = take(qmoe::permute_scratch_bytes(A, static_cast<int>(p->num_experts)));
  w.h = take(rows * p->inter_size * act);
  w.y = reinterpret_cast<float*>(take(rows * p->hidden_size * 4));
  if (use_i8_dot(p)) {
    const int64_t nbh = (p->hidden_size + p->block_size - 1) / p->block_size;
    const int64_t nbi = (p->inter_size + p->block_size - 1) / p->block_size;
    w.xc = reinterpret_cast<int8_t*>(take(p->num_tokens * p->hidden_size));
    w.xf = reinterpret_cast<float*>(take(p->num_tokens * nbh * 4));
    w.hc = reinterpret_cast<int8_t*>(take(rows * p->inter_size));
    w.hf = reinterpret_cast<float*>(take(rows * nbi * 4));
  } else if (p->compute_mode == QMOE_COMPUTE_INT8) {
    w.xq = take(p->num_tokens * p->hidden_size * act);
  }
  if (use_xsum(p)) w.xsum = reinterpret_cast<float*>(take(p->num_tokens * 4));
  if (use_hpart(p)) {
    w.hpart = reinterpret_cast<float*>(take(rows * hpart_blocks(p) * 4));
    w.hsum = reinterpret_cast<float*>(take(rows * 4));
  }
  if (use_h16(p)) {
    w.x16 = take(p->num_tokens * p->hidden_size * 2);
    w.xlift = reinterpret_cast<int32_t*>(take(p->num_tokens * 4));
    w.h16 = take(rows * p->inter_size * 2);
    w.hlift = reinterpret_cast<int32_t*>(take(rows * 4));
    w.w1lift = reinterpret_cast<int32_t*>(take(p->num_experts * n1_rows(p) * 4));
    if (has_fc3(p)) w.w3lift = reinterpret_cast<int32_t*>(take(p->num_experts * p->inter_size * 4));
    w.w2lift = reinterpret_cast<int32_t*>(take(p->num_experts * p->hidden_size * 4));
  }
  w.bytes = off;
  return w;
}

// Tiled layout of stack `which`; false when the stack does not exist for these parameters.
bool pack_args(const qmoe_params* p, int32_t which, qmoe::PackArgs& a) {
  a.E = static_cast<int>(p->num_experts);
  a.bits = p->expert_weight_bits;
  a.fusion = 0;
  a.S = 1;
  if (which == QMOE_FC1) {
    a.K = static_cast<int>(p->hidden_size);
    a.rows = static_cast<int>(p->inter_size);
    a.N = static_cast<int>(n1_rows(p));
    if (swiglu(p) && p->swiglu_fusion != 0) {
      a.S = 2;
      a.fusion = p->swiglu_fusion;
    }
  } else if (which == QMOE_FC3) {
    if (!has_fc3(p)) return false;
    a.K = static_cast<int>(p->hidden_size);
    a.rows = a.N = static_cast<int>(p->inter_size);
  } else if (which == QMOE_FC2) {
    a.K = static_cast<int>(p->inter_size);
    a.rows = a.N = static_cast<int>(p->hidden_size);
  } else {
    return false;
  }
  const int ssk = p->expert_weight_bits == 4 ? 128 : 64;
  a.natural = p->scale_dtype == QMOE_E8M0;
  a.NB = (a.rows + 15) / 16;
  a.KT = (a.K + ssk - 1) / ssk;
  return true;
}

size_t packed_bytes(const qmoe::PackArgs& a) {
  return static_cast<size_t>(a.E) * a.S * a.NB * a.KT * 1024;
}

qmoe::GemmArgs gemm_args(const qmoe_params* p) {
  qmoe::GemmArgs g{};
  g.topk = static_cast<int>(p->k);
  g.bs = p->block_size;
  g.bs_shift = 0;
  while (g.bs > 0 && (1 << g.bs_shift) < g.bs) ++g.bs_shift;
  g.fusion = p->swiglu_fusion;
  // activation code of the kernels: 1 identity, 2 relu, 3 silu, 4 gelu (erf), 5 gelu (tanh)
  g.act = p->activation == QMOE_ACT_GELU ? (p->gelu_mode ? 5 : 4) : p->activation;
  g.alpha = p->swiglu_alpha;
  g.beta = p->swiglu_beta;
  g.limit = (p->swiglu_limit > 0.f) ? p->swiglu_limit : INFINITY;
  g.inter = static_cast<int>(p->inter_size);
  g.M = tile_m_of(p);
  g.packed = p->weight_layout == QMOE_LAYOUT_TILES;
  g.mx = p->scale_dtype == QMOE_E8M0;
  return g;
}

// Tile counts of the tiled layout for a GEMM over K with `rows` rows per stream.
void set_tiles(const qmoe_params* p, qmoe::GemmArgs& g, int rows) {
  const int ssk = p->expert_weight_bits == 4 ? 128 : 64;
  g.kt = (g.K + ssk - 1) / ssk;
  g.nbk = (rows + 15) / 16;
}

// Kernel variant from the element types and the tile height (itself chosen from shapes).
hipError_t launch_gemm(const qmoe_params* p, const qmoe::GemmArgs& g, int mode, hipStream_t s) {
  const bool sbf = p->scale_dtype == QMOE_BF16;
  const int bits = p->expert_weight_bits;
  if (g.afac) return qmoe::launch_gemm_i8_prefill(g, mode, bits, sbf, max_tiles_of(p), s);
  if (g.alift) return qmoe::launch_gemm_h16_prefill(g, mode, max_tiles_of(p), s);
  if (p->act_dtype != QMOE_BF16) return qmoe::launch_gemm_f32(g, mode, bits, sbf, max_tiles_of(p), s);
  if (tile_m_of(p) == 128) return qmoe::launch_gemm_bf16_prefill(g, mode, bits, sbf, max_tiles_of(p), s);
  return qmoe::launch_gemm_bf16(g, mode, bits, sbf, max_tiles_of(p), s);
}

qmoe_status run_fc1(const qmoe_params* p, const void* x, const int32_t* sorted_assign,
                    const int32_t* tiles, const int32_t* num_tiles, const float* topk_w,
                    qmoe_stack fc1, qmoe_stack fc3, void* h, hipStream_t s,
                    const float* xfac = nullptr, const float* xsum = nullptr,
                    const Workspace* h16 = nullptr, float* hpart = nullptr) {
  qmoe::GemmArgs g = gemm_args(p);
  g.a = x;
  g.afac = xfac;
  g.xsum = xsum;
  if (hpart) {
    g.hpart = hpart;
    g.hpart_stride = hpart_blocks(p);
  }
  if (h16) {
    g.a = h16->x16;
    g.alift = h16->xlift;
    g.wlift = h16->w1lift;
    g.wlift3 = h16->w3lift;
  }
  g.sorted_assign = sorted_assign;
  g.row_w = p->apply_router_weight_on_input ? topk_w : nullptr;
  g.tile_list = tiles;
  g.num_tiles = num_tiles;
  g.w = static_cast<const uint8_t*>(fc1.weights);
  g.s = fc1.scales;
  g.b = fc1.bias;
  if (has_fc3(p)) {
    g.w3 = static_cast<const uint8_t*>(fc3.weights);
    g.s3 = fc3.scales;
    g.b3 = fc3.bias;
  }
  g.out = h;
  g.K = static_cast<int>(p->hidden_size);
  g.a_rows = p->num_tokens;
  g.N = static_cast<int>(n1_rows(p));
  g.ncols = static_cast<int>(p->inter_size);
  g.nb = p->block_size ? static_cast<int>((p->hidden_size + p->block_size - 1) / p->block_size) : 0;
  set_tiles(p, g, static_cast<int>(p->inter_size));
  const int mode = swiglu(p) ? qmoe::kModeSwiglu : qmoe::kModePlainAct;
  return device_status(launch_gemm(p, g, mode, s), "fc1 launch");
}

// The single-expert linear layer: the fc1-side GEMM over the rows of x in consecutive
// tiles, plain activation epilogue, output rows stored only for real rows.
qmoe_status run_linear(const qmoe_params* p, const void* x, qmoe_stack w, void* y, hipStream_t s) {
  qmoe::GemmArgs g = gemm_args(p);
  g.a = x;
  g.linear = 1;
  g.w = static_cast<const uint8_t*>(w.weights);
  g.s = w.scales;
  g.b = w.bias;
  g.out = y;
  g.K = static_cast<int>(p->hidden_size);
  g.a_rows = p->num_tokens;
  g.N = static_cast<int>(p->inter_size);
  g.ncols = static_cast<int>(p->inter_size);
  g.nb = p->block_size ? static_cast<int>((p->hidden_size + p->block_size - 1) / p->block_size) : 0;
  set_tiles(p, g, static_cast<int>(p->inter_size));
  return device_status(launch_gemm(p, g, qmoe::kModePlainAct, s), "linear launch");
}

qmoe_status run_fc2(const qmoe_params* p, const void* h, const int32_t* tiles,
                    const int32_t* num_tiles, qmoe_stack fc2, float* y, hipStream_t s,
                    const float* hfac = nullptr, const Workspace* h16 = nullptr,
                    const float* hsum = nullptr) {
  qmoe::GemmArgs g = gemm_args(p);
  g.a = h;
  g.afac = hfac;
  g.xsum = hsum;
  if (h16) {
    g.a = h16->h16;
    g.alift = h16->hlift;
    g.wlift = h16->w2lift;
  }
  g.tile_list = tiles;
  g.num_tiles = num_tiles;
  g.w = static_cast<const uint8_t*>(fc2.weights);
  g.s = fc2.scales;
  g.b = fc2.bias;
  g.out = y;
  g.K = static_cast<int>(p->inter_size);
  g.a_rows = max_rows_of(p);
  g.N = static_cast<int>(p->hidden_size);
  g.ncols = static_cast<int>(p->hidden_size);
  g.nb = p->block_size ? static_cast<int>((p->inter_size + p->block_size - 1) / p->block_size) : 0;
  set_tiles(p, g, static_cast<int>(p->hidden_size));
  return device_status(launch_gemm(p, g, qmoe::kModeFc2, s), "fc2 launch");
}

qmoe_status need(const void* ptr, const char* name) {
  if (!ptr) return fail(QMOE_ERR_UNBOUND, "%s is NULL", name);
  return QMOE_OK;
}

#define QMOE_TRY(expr)                  \
  do {                                  \
    qmoe_status st__ = (expr);          \
    if (st__ != QMOE_OK) return st__;   \
  } while (0)

qmoe_status check_stack(const qmoe_stack& st, const char* name) {
  char buf[64];
  snprintf(buf, sizeof(buf), "%s.weights", name);
  QMOE_TRY(need(st.weights, buf));
  snprintf(buf, sizeof(buf), "%s.scales", name);
  QMOE_TRY(need(st.scales, buf));
  return QMOE_OK;
}

}  // namespace

extern "C" {

qmoe_status qmoe_validate(const qmoe_params* p) { return validate(p); }

int32_t qmoe_tile_m(const qmoe_params* p) { return p ? tile_m_of(p) : 0; }

int64_t qmoe_max_rows(const qmoe_params* p) { return p ? max_rows_of(p) : 0; }

int64_t qmoe_max_tiles(const qmoe_params* p) { return p ? max_tiles_of(p) : 0; }

size_t qmoe_permute_scratch_size(const qmoe_params* p) {
  if (!p) return 0;
  return qmoe::permute_scratch_bytes(p->num_tokens * p->k, static_cast<int>(p->num_experts));
}

size_t qmoe_workspace_size(const qmoe_params* p) {
  if (validate(p) != QMOE_OK) return 0;
  return carve(p, nullptr).bytes;
}

qmoe_status qmoe_route(const qmoe_params* p, const void* router_logits, int32_t* topk_ids,
                       float* topk_w, void* stream) {
  QMOE_TRY(validate(p));
  if (p->num_tokens == 0) return ok();
  QMOE_TRY(need(router_logits, "router_logits"));
  QMOE_TRY(need(topk_ids, "topk_ids"));
  QMOE_TRY(need(topk_w, "topk_w"));
  return device_status(
      qmoe::launch_route(router_logits, p->act_dtype == QMOE_BF16, static_cast<int>(p->num_tokens),
                         static_cast<int>(p->num_experts), static_cast<int>(p->k),
                         p->normalize_routing_weights, route_opts(p), topk_ids, topk_w,
                         static_cast<hipStream_t>(stream)),
      "route launch");
}

qmoe_status qmoe_permute(const qmoe_params* p, const int32_t* topk_ids, int32_t* counts,
                         int32_t* padded_offsets, int32_t* sorted_assign, int32_t* assign_pos,
                         int32_t* tile_list, int32_t* num_tiles, void* scratch,
                         size_t scratch_bytes, void* stream) {
  QMOE_TRY(validate(p));
  if (p->num_tokens == 0) return ok();
  QMOE_TRY(need(topk_ids, "topk_ids"));
  QMOE_TRY(need(counts, "counts"));
  QMOE_TRY(need(padded_offsets, "padded_offsets"));
  QMOE_TRY(need(sorted_assign, "sorted_assign"));
  QMOE_TRY(need(assign_pos, "assign_pos"));
  QMOE_TRY(need(tile_list, "tile_list"));
  QMOE_TRY(need(num_tiles, "num_tiles"));
  const size_t want = qmoe_permute_scratch_size(p);
  if (want > 0) {
    QMOE_TRY(need(scratch, "scratch"));
    if (scratch_bytes < want)
      return fail(QMOE_ERR_INVALID, "permute scratch %zu bytes < %zu", scratch_bytes, want);
  }
  return device_status(
      qmoe::launch_permute(topk_ids, p->num_tokens * p->k, static_cast<int>(p->num_experts),
                           tile_m_of(p), counts, padded_offsets, sorted_assign, assign_pos,
                           tile_list, num_tiles, scratch, static_cast<hipStream_t>(stream)),
      "permute launch");
}

qmoe_status qmoe_grouped_gemm_fc1_swiglu(const qmoe_params* p, const void* x,
                                         const int32_t* sorted_assign, const int32_t* tile_list,
                                         const int32_t* num_tiles, const float* topk_w,
                                         qmoe_stack fc1, qmoe_stack fc3, void* h, void* stream) {
  QMOE_TRY(validate(p));
  if (p->num_tokens == 0) return ok();
  QMOE_TRY(need(x, "x"));
  QMOE_TRY(need(sorted_assign, "sorted_assign"));
  QMOE_TRY(need(tile_list, "tile_list"));
  QMOE_TRY(need(num_tiles, "num_tiles"));
  QMOE_TRY(check_stack(fc1, "fc1"));
  if (has_fc3(p)) QMOE_TRY(check_stack(fc3, "fc3"));
  QMOE_TRY(need(h, "h"));
  if (p->apply_router_weight_on_input) QMOE_TRY(need(topk_w, "topk_w"));
  return run_fc1(p, x, sorted_assign, tile_list, num_tiles, topk_w, fc1, fc3, h,
                 static_cast<hipStream_t>(stream));
}

qmoe_status qmoe_grouped_gemm_fc2(const qmoe_params* p, const void* h, const int32_t* tile_list,
                                  const int32_t* num_tiles, qmoe_stack fc2, float* y,
                                  void* stream) {
  QMOE_TRY(validate(p));
  if (p->num_tokens == 0) return ok();
  QMOE_TRY(need(h, "h"));
  QMOE_TRY(need(tile_list, "tile_list"));
  QMOE_TRY(need(num_tiles, "num_tiles"));
  QMOE_TRY(check_stack(fc2, "fc2"));
  QMOE_TRY(need(y, "y"));
  return run_fc2(p, h, tile_list, num_tiles, fc2, y, static_cast<hipStream_t>(stream));
}

qmoe_status qmoe_combine(const qmoe_params* p, const float* y, const int32_t* assign_pos,
                         const float* topk_w, const void* shared_output, void* output,
                         void* stream) {
  QMOE_TRY(validate(p));
  if (p->num_tokens == 0) return ok();
  QMOE_TRY(need(y, "y"));
  QMOE_TRY(need(assign_pos, "assign_pos"));
  QMOE_TRY(need(topk_w, "topk_w"));
  QMOE_TRY(need(output, "output"));
  return device_status(
      qmoe::launch_combine(y, assign_pos, topk_w, shared_output, output,
                           p->act_dtype == QMOE_BF16, static_cast<int>(p->num_tokens),
                           static_cast<int>(p->hidden_size), static_cast<int>(p->k),
                           combine_opts(p), static_cast<hipStream_t>(stream)),
      "combine launch");
}

qmoe_status qmoe_workspace_layout_of(const qmoe_params* p, qmoe_workspace_layout* out) {
  QMOE_TRY(validate(p));
  QMOE_TRY(need(out, "out"));
  const Workspace w = carve(p, nullptr);
  // carve() on a null base yields the offsets themselves (base + offset with base = 0)
  auto off = [](const void* ptr) { return static_cast<size_t>(reinterpret_cast<uintptr_t>(ptr)); };
  *out = qmoe_workspace_layout{};
  out->topk_ids = off(w.topk_ids);
  out->topk_w = off(w.topk_w);
  out->counts = off(w.counts);
  out->padded_offsets = off(w.offsets);
  out->sorted_assign = off(w.sorted_assign);
  out->assign_pos = off(w.assign_pos);
  out->tile_list = off(w.tiles);
  out->num_tiles = off(w.num_tiles);
  out->permute_scratch = off(w.perm_scratch);
  out->h = off(w.h);
  out->y = off(w.y);
  out->xq = (p->compute_mode == QMOE_COMPUTE_INT8 && !use_i8_dot(p)) ? off(w.xq) : 0;
  const bool i8 = use_i8_dot(p);
  out->xcodes = i8 ? off(w.xc) : 0;
  out->xfactors = i8 ? off(w.xf) : 0;
  out->hcodes = i8 ? off(w.hc) : 0;
  out->hfactors = i8 ? off(w.hf) : 0;
  out->xsum = use_xsum(p) ? off(w.xsum) : 0;
  out->hpart = use_hpart(p) ? off(w.hpart) : 0;
  const bool h16 = use_h16(p);
  out->x16 = h16 ? off(w.x16) : 0;
  out->xlift = h16 ? off(w.xlift) : 0;
  out->h16 = h16 ? off(w.h16) : 0;
  out->hlift = h16 ? off(w.hlift) : 0;
  out->total = w.bytes;
  out->fused_routing = qmoe::route_permute_fits(p->num_tokens, p->num_tokens * p->k,
                                                p->num_experts, p->k) ? 1 : 0;
  return ok();
}

qmoe_status qmoe_forward(const qmoe_params* p, const void* input, const void* router_logits,
                         qmoe_stack fc1, qmoe_stack fc2, qmoe_stack fc3,
                         const void* shared_output, void* output, void* workspace,
                         size_t workspace_bytes, void* stream) {
  QMOE_TRY(validate(p));
  if (p->num_tokens == 0) return ok();
  QMOE_TRY(need(input, "input"));
  QMOE_TRY(need(router_logits, "router_probs"));
  QMOE_TRY(check_stack(fc1, "fc1"));
  QMOE_TRY(check_stack(fc2, "fc2"));
  if (has_fc3(p)) QMOE_TRY(check_stack(fc3, "fc3"));
  QMOE_TRY(need(output, "output"));
  QMOE_TRY(need(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(QMOE_ERR_INVALID, "workspace must be 256-byte aligned");
  Workspace w = carve(p, static_cast<char*>(workspace));
  if (workspace_bytes < w.bytes)
    return fail(QMOE_ERR_INVALID, "workspace %zu bytes < %zu", workspace_bytes, w.bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t A = p->num_tokens * p->k;
  if (qmoe::route_permute_fits(p->num_tokens, A, p->num_experts, p->k)) {
    QMOE_TRY(device_status(
        qmoe::launch_route_permute(router_logits, p->act_dtype == QMOE_BF16,
                                   static_cast<int>(p->num_tokens), static_cast<int>(p->num_experts),
                                   static_cast<int>(p->k), p->normalize_routing_weights,
                                   route_opts(p), tile_m_of(p), w.topk_w, w.counts, w.offsets,
                                   w.sorted_assign, w.assign_pos, w.tiles, w.num_tiles, s),
        "route+permute launch"));
  } else {
    QMOE_TRY(device_status(
        qmoe::launch_route(router_logits, p->act_dtype == QMOE_BF16, static_cast<int>(p->num_tokens),
                           static_cast<int>(p->num_experts), static_cast<int>(p->k),
                           p->normalize_routing_weights, route_opts(p), w.topk_ids, w.topk_w, s),
        "route launch"));
    QMOE_TRY(device_status(
        qmoe::launch_permute(w.topk_ids, A, static_cast<int>(p->num_experts), tile_m_of(p), w.counts,
                             w.offsets, w.sorted_assign, w.assign_pos, w.tiles, w.num_tiles,
                             w.perm_scratch, s),
        "permute launch"));
  }
  const bool int8 = p->compute_mode == QMOE_COMPUTE_INT8;
  const bool abf = p->act_dtype == QMOE_BF16;
  const void* x = input;
  if (use_i8_dot(p)) {
    // the int8 dot: x and h as int8 codes with their block factors
    const int H = static_cast<int>(p->hidden_size), I = static_cast<int>(p->inter_size);
    QMOE_TRY(device_status(qmoe::launch_quantize_codes(input, w.xc, w.xf, p->num_tokens, H,
                                                       p->block_size, nullptr, 0, s),
                           "quantize x launch"));
    QMOE_TRY(run_fc1(p, w.xc, w.sorted_assign, w.tiles, w.num_tiles, w.topk_w, fc1, fc3, w.h, s,
                     w.xf));
    QMOE_TRY(device_status(qmoe::launch_quantize_codes(w.h, w.hc, w.hf, max_rows_of(p), I,
                                                       p->block_size, w.num_tiles, 128, s),
                           "quantize h launch"));
    QMOE_TRY(run_fc2(p, w.hc, w.tiles, w.num_tiles, fc2, w.y, s, w.hf));
    QMOE_TRY(device_status(
        qmoe::launch_combine(w.y, w.assign_pos, w.topk_w, shared_output, output,
                             p->act_dtype == QMOE_BF16, static_cast<int>(p->num_tokens),
                             static_cast<int>(p->hidden_size), static_cast<int>(p->k),
                             combine_opts(p), s),
        "combine launch"));
    return ok();
  }
  if (int8) {
    QMOE_TRY(device_status(qmoe::launch_quantize_blocks(input, w.xq, abf, p->num_tokens,
                                                        static_cast<int>(p->hidden_size),
                                                        p->block_size, nullptr, 0, s),
                           "quantize x launch"));
    x = w.xq;
  }
  if (use_h16(p)) {
    // the fp16 block-scale path: lifts of the weight rows' scales and x in fp16 (one
    // launch), fc1, h in fp16 (the rows of the tiles in use), fc2
    const int H = static_cast<int>(p->hidden_size), I = static_cast<int>(p->inter_size);
    const int nbh = (H + p->block_size - 1) / p->block_size;
    const int nbi = (I + p->block_size - 1) / p->block_size;
    const void* sc[3] = {fc1.scales, has_fc3(p) ? fc3.scales : nullptr, fc2.scales};
    int32_t* const lifts[3] = {w.w1lift, w.w3lift, w.w2lift};
    const int64_t srows[3] = {p->num_experts * n1_rows(p), p->num_experts * I, p->num_experts * H};
    const int snb[3] = {nbh, nbh, nbi};
    QMOE_TRY(device_status(qmoe::launch_prep_f16(sc, lifts, srows, snb, input, w.x16, w.xlift,
                                                 p->num_tokens, H, s),
                           "fp16 operands launch"));
    QMOE_TRY(run_fc1(p, input, w.sorted_assign, w.tiles, w.num_tiles, w.topk_w, fc1, fc3, w.h, s,
                     nullptr, nullptr, &w));
    QMOE_TRY(device_status(qmoe::launch_rows_to_f16(w.h, w.h16, w.hlift, max_rows_of(p), I, w.num_tiles,
                                                    128, s),
                           "h to fp16 launch"));
    QMOE_TRY(run_fc2(p, w.h, w.tiles, w.num_tiles, fc2, w.y, s, nullptr, &w));
    QMOE_TRY(device_status(
        qmoe::launch_combine(w.y, w.assign_pos, w.topk_w, shared_output, output, true,
                             static_cast<int>(p->num_tokens), H, static_cast<int>(p->k),
                             combine_opts(p), s),
        "combine launch"));
    return ok();
  }
  if (use_xsum(p))
    QMOE_TRY(device_status(qmoe::launch_rowsum(x, w.xsum, p->num_tokens,
                                               static_cast<int>(p->hidden_size), s),
                           "row sum launch"));
  QMOE_TRY(run_fc1(p, x, w.sorted_assign, w.tiles, w.num_tiles, w.topk_w, fc1, fc3, w.h, s,
                   nullptr, w.xsum, nullptr, w.hpart));
  if (int8)
    QMOE_TRY(device_status(qmoe::launch_quantize_blocks(w.h, w.h, abf, max_rows_of(p),
                                                        static_cast<int>(p->inter_size),
                                                        p->block_size, w.num_tiles,
                                                        static_cast<int>(tile_m_of(p)), s),
                           "quantize h launch"));
  if (use_hpart(p))
    QMOE_TRY(device_status(qmoe::launch_partsum(w.hpart, w.hsum, max_rows_of(p), hpart_blocks(p),
                                                w.num_tiles, 128, s),
                           "h row sum launch"));
  QMOE_TRY(run_fc2(p, w.h, w.tiles, w.num_tiles, fc2, w.y, s, nullptr, nullptr, w.hsum));
  QMOE_TRY(device_status(
      qmoe::launch_combine(w.y, w.assign_pos, w.topk_w, shared_output, output,
                           p->act_dtype == QMOE_BF16, static_cast<int>(p->num_tokens),
                           static_cast<int>(p->hidden_size), static_cast<int>(p->k),
                           combine_opts(p), s),
      "combine launch"));
  return ok();
}

size_t qmoe_packed_stack_size(const qmoe_params* p, int32_t which) {
  if (validate_for_pack(p) != QMOE_OK) return 0;
  qmoe::PackArgs a{};
  if (!pack_args(p, which, a)) return 0;
  return packed_bytes(a);
}

qmoe_status qmoe_pack_stack(const qmoe_params* p, int32_t which, const void* weights,
                            void* packed, void* stream) {
  QMOE_TRY(validate_for_pack(p));
  qmoe::PackArgs a{};
  if (!pack_args(p, which, a))
    return fail(QMOE_ERR_INVALID, "stack %d does not exist for these parameters", which);
  QMOE_TRY(need(weights, "weights"));
  QMOE_TRY(need(packed, "packed"));
  if (reinterpret_cast<uintptr_t>(packed) % 256)
    return fail(QMOE_ERR_INVALID, "packed must be 256-byte aligned");
  const size_t nbytes = packed_bytes(a);
  const size_t src_bytes = static_cast<size_t>(a.E) * a.N * a.K * a.bits / 8;
  const char* w0 = static_cast<const char*>(weights);
  const char* p0 = static_cast<const char*>(packed);
  if (p0 < w0 + src_bytes && w0 < p0 + nbytes)
    return fail(QMOE_ERR_INVALID, "packed overlaps weights");
  return device_status(qmoe::launch_pack_stack(static_cast<const uint8_t*>(weights),
                                               static_cast<uint8_t*>(packed), a,
                                               static_cast<hipStream_t>(stream)),
                       "pack launch");
}

qmoe_status qmoe_linear_woq(const qmoe_params* p, const void* x, qmoe_stack w, void* y,
                            void* stream) {
  QMOE_TRY(validate(p));
  if (p->num_experts != 1 || p->k != 1)
    return fail(QMOE_ERR_INVALID, "a linear layer has num_experts 1 and k 1 (got %lld, %lld)",
                (long long)p->num_experts, (long long)p->k);
  if (swiglu(p))
    return fail(QMOE_ERR_INVALID, "a linear layer's activation is identity, relu, silu or gelu");
  if (p->apply_router_weight_on_input)
    return fail(QMOE_ERR_INVALID, "a linear layer has no routing weight to apply");
  if (p->num_tokens == 0) return ok();
  QMOE_TRY(need(x, "x"));
  QMOE_TRY(check_stack(w, "weight"));
  QMOE_TRY(need(y, "y"));
  return run_linear(p, x, w, y, static_cast<hipStream_t>(stream));
}

qmoe_status qmoe_quantize_act(const qmoe_params* p, const void* in, int64_t rows, int64_t cols,
                              void* out, void* stream) {
  QMOE_TRY(validate(p));
  if (p->block_size == 0)
    return fail(QMOE_ERR_INVALID, "the int8 activation tier needs block_size > 0");
  if (rows < 0 || cols < 1 || cols >= (int64_t(1) << 31))
    return fail(QMOE_ERR_SHAPE, "rows %lld, cols %lld", (long long)rows, (long long)cols);
  if (rows == 0) return ok();
  QMOE_TRY(need(in, "in"));
  QMOE_TRY(need(out, "out"));
  return device_status(qmoe::launch_quantize_blocks(in, out, p->act_dtype == QMOE_BF16, rows,
                                                    static_cast<int>(cols), p->block_size, nullptr, 0,
                                                    static_cast<hipStream_t>(stream)),
                       "quantize launch");
}

qmoe_status qmoe_time_next_gemm(void* start_event, void* stop_event) {
  qmoe::set_gemm_timing(static_cast<hipEvent_t>(start_event),
                        static_cast<hipEvent_t>(stop_event));
  return ok();
}

const char* qmoe_last_error(void) { return g_error.c_str(); }

}  // extern "C"
