// C entry points: argument checks on the host, then kernel launches.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "gemm_common.h"

namespace moe {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

moe_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status launch_route(const float*, const float*, int64_t, const moe_route_params*, int32_t*, float*, hipStream_t);
size_t permute_ws_bytes(int64_t R, int E);
moe_status launch_permute(const int32_t*, int64_t, int, int, int32_t*, int32_t*, int32_t*, void*, hipStream_t);
bool route_permute_fits(int64_t T, int top_k);
size_t route_gemv_ws_bytes(int64_t T, int E);
moe_status launch_route_gemv(const void*, const float*, const float*, int64_t, int, const moe_route_params*, int32_t*,
                             float*, void*, hipStream_t);
moe_status launch_route_permute(const float*, const float*, int64_t, const moe_route_params*, int32_t*, float*, int32_t*,
                                int32_t*, int32_t*, uint32_t*, hipStream_t);
moe_status launch_combine(const void*, const int32_t*, const float*, const void*, int64_t, int, int, void*, hipStream_t);
moe_status launch_transcode(const uint8_t*, const uint8_t*, int64_t, int, int, uint8_t*, float*, int64_t*, hipStream_t);
moe_status launch_quant(const void*, int64_t, int, float, uint8_t*, uint8_t*, void*, hipStream_t);
moe_status launch_tile(int, int64_t, int, int, const uint8_t*, const uint8_t*, uint8_t*, uint8_t*, hipStream_t);
moe_status launch_gemm_decode(const GemmArgs&, bool swiglu, int wf, bool a_nv, int64_t rows, hipStream_t);
moe_status launch_gemm_prefill(const GemmArgs&, bool swiglu, int wf, bool a_nv, int64_t rows, hipStream_t);
moe_status launch_gemm_scaled(const GemmArgs&, bool swiglu, bool planes, bool w_nv, hipStream_t);
moe_status launch_quant_mxfp8(const void*, int64_t, int, uint8_t*, uint8_t*, hipStream_t);
moe_status launch_saliency(const float*, int64_t, int, const int32_t*, int, const int32_t*, const float*, double*,
                           int64_t*, hipStream_t);
moe_status launch_quant_planes(const void*, int64_t, int, float, uint8_t*, uint8_t*, hipStream_t);
moe_status launch_compact(const uint8_t*, const uint8_t*, int64_t, int, int, uint8_t*, float*, int64_t*, hipStream_t);

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static bool is_pow2_float(float g) {
  if (!(g > 0.0f)) return false;
  int e;
  float m = frexpf(g, &e);
  return m == 0.5f;
}

#define MOE_CHECK(cond, ...)      \
  do {                            \
    if (!(cond)) {                \
      moe::set_error(__VA_ARGS__); \
      return MOE_ERR_INVALID;     \
    }                             \
  } while (0)

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

const char* moe_version(void) { return "moe_fp4 gfx950 1.0"; }

static moe_status check_route(const moe_route_params* p, int64_t T) {
  MOE_CHECK(p != nullptr, "moe_route: params is NULL");
  MOE_CHECK(T >= 0, "moe_route: T < 0");
  const int E = p->num_experts;
  MOE_CHECK(E >= 2 && E <= 256, "moe_route: num_experts %d outside [2, 256]", E);
  MOE_CHECK(p->n_group >= 1 && p->n_group <= 64 && E % p->n_group == 0, "moe_route: bad n_group %d", p->n_group);
  MOE_CHECK(E / p->n_group >= 2, "moe_route: groups need >= 2 experts");
  MOE_CHECK(p->topk_group >= 1 && p->topk_group <= p->n_group, "moe_route: bad topk_group %d", p->topk_group);
  MOE_CHECK(p->top_k >= 1 && p->top_k <= 16 && p->top_k <= p->topk_group * (E / p->n_group),
            "moe_route: bad top_k %d", p->top_k);
  return MOE_OK;
}

moe_status moe_route(const float* logits, const float* correction_bias, int64_t T, const moe_route_params* p,
                     int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  g_err[0] = 0;
  const moe_status st = check_route(p, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  MOE_CHECK(logits && topk_ids && topk_weights, "moe_route: NULL pointer");
  return launch_route(logits, correction_bias, T, p, topk_ids, topk_weights, stream);
}

size_t moe_permute_workspace_bytes(int64_t T, int32_t top_k, int32_t num_experts) {
  if (T < 0 || top_k <= 0 || num_experts <= 0) return 0;
  return permute_ws_bytes(T * top_k, num_experts);
}

moe_status moe_permute(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t num_experts,
                       int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_rows, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(T >= 0 && top_k >= 1, "moe_permute: bad T / top_k");
  MOE_CHECK(num_experts >= 1 && num_experts <= 1024, "moe_permute: num_experts %d outside [1, 1024]", num_experts);
  MOE_CHECK(T * (int64_t)top_k < ((int64_t)1 << 31), "moe_permute: too many slots");
  MOE_CHECK(expert_offsets != nullptr, "moe_permute: expert_offsets is NULL");
  if (T > 0) MOE_CHECK(topk_ids && sorted_slots && slot_rows, "moe_permute: NULL pointer");
  size_t need = permute_ws_bytes(T * top_k, num_experts);
  if (T * (int64_t)top_k > 2048) {
    if (workspace_bytes < need || workspace == nullptr) {
      set_error("moe_permute: workspace %zu bytes < %zu", workspace_bytes, need);
      return MOE_ERR_WORKSPACE;
    }
  }
  return launch_permute(topk_ids, T, top_k, num_experts, expert_offsets, sorted_slots, slot_rows, workspace, stream);
}

moe_status moe_route_permute(const float* logits, const float* correction_bias, int64_t T, const moe_route_params* p,
                             int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets, int32_t* sorted_slots,
                             int32_t* slot_rows, uint32_t* counter, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  g_err[0] = 0;
  const moe_status st = check_route(p, T);
  if (st != MOE_OK) return st;
  if (!route_permute_fits(T, p->top_k)) {
    // two launches; every argument of both is checked before the first
    MOE_CHECK(expert_offsets != nullptr, "moe_route_permute: expert_offsets is NULL");
    if (T > 0) {
      MOE_CHECK(logits && topk_ids && topk_weights && sorted_slots && slot_rows, "moe_route_permute: NULL pointer");
      MOE_CHECK(T * (int64_t)p->top_k < ((int64_t)1 << 31), "moe_route_permute: too many slots");
      const size_t need = permute_ws_bytes(T * p->top_k, p->num_experts);
      if (workspace_bytes < need || workspace == nullptr) {
        set_error("moe_route_permute: workspace %zu bytes < %zu", workspace_bytes, need);
        return MOE_ERR_WORKSPACE;
      }
      const moe_status rs = launch_route(logits, correction_bias, T, p, topk_ids, topk_weights, stream);
      if (rs != MOE_OK) return rs;
    }
    return moe_permute(topk_ids, T, p->top_k, p->num_experts, expert_offsets, sorted_slots, slot_rows, workspace,
                       workspace_bytes, stream);
  }
  MOE_CHECK(logits && topk_ids && topk_weights && expert_offsets && sorted_slots && slot_rows && counter,
            "moe_route_permute: NULL pointer");
  MOE_CHECK(((uintptr_t)counter & 3) == 0, "moe_route_permute: counter not 4-byte aligned");
  return launch_route_permute(logits, correction_bias, T, p, topk_ids, topk_weights, expert_offsets, sorted_slots,
                              slot_rows, counter, stream);
}

size_t moe_route_gemv_workspace_bytes(int64_t T, int32_t num_experts) {
  if (T < 0 || num_experts <= 0) return 0;
  return route_gemv_ws_bytes(T, num_experts);
}

moe_status moe_route_gemv(const void* x, const float* gate_weight, const float* correction_bias, int64_t T,
                          int32_t hidden, const moe_route_params* p, int32_t* topk_ids, float* topk_weights,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  const moe_status st = check_route(p, T);
  if (st != MOE_OK) return st;
  MOE_CHECK(hidden >= 512 && hidden % 512 == 0, "moe_route_gemv: hidden %d must be a positive multiple of 512", hidden);
  MOE_CHECK(T <= (int64_t)65535 * 16, "moe_route_gemv: T > 1048560");
  if (T == 0) return MOE_OK;
  MOE_CHECK(x && gate_weight && topk_ids && topk_weights, "moe_route_gemv: NULL pointer");
  MOE_CHECK(aligned16(x) && aligned16(gate_weight), "moe_route_gemv: x and gate_weight must be 16-byte aligned");
  const size_t need = route_gemv_ws_bytes(T, p->num_experts);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) {
    set_error("moe_route_gemv: workspace %zu bytes < %zu (or NULL / unaligned)", workspace_bytes, need);
    return MOE_ERR_WORKSPACE;
  }
  return launch_route_gemv(x, gate_weight, correction_bias, T, hidden, p, topk_ids, topk_weights, workspace, stream);
}

static moe_status check_weights(const moe_fp4_weights* w, const char* name) {
  MOE_CHECK(w != nullptr, "moe_fp4_grouped_gemm: %s is NULL", name);
  MOE_CHECK(w->format == MOE_FP4_MX || w->format == MOE_FP4_NV || w->format == MOE_FP4_MXC,
            "moe_fp4_grouped_gemm: %s bad format", name);
  MOE_CHECK(w->num_experts >= 1 && w->n >= 16 && w->k >= 128, "moe_fp4_grouped_gemm: %s bad shape", name);
  MOE_CHECK(w->packed && w->scale, "moe_fp4_grouped_gemm: %s NULL data", name);
  MOE_CHECK(aligned16(w->packed), "moe_fp4_grouped_gemm: %s codes not 16-byte aligned", name);
  if (w->format != MOE_FP4_MX)
    MOE_CHECK(w->global_scale != nullptr, "moe_fp4_grouped_gemm: %s NV / MXC without global scales", name);
  MOE_CHECK((w->flags & ~(MOE_FP4_SCALES_POW2 | MOE_FP4_TILED | MOE_FP4_MX_EXACT)) == 0,
            "moe_fp4_grouped_gemm: %s unknown flags 0x%x", name, w->flags);
  MOE_CHECK(w->format == MOE_FP4_NV || (w->flags & (MOE_FP4_SCALES_POW2 | MOE_FP4_MX_EXACT)) == 0,
            "moe_fp4_grouped_gemm: %s scale flags are for NV weights", name);
  if (w->k % 128 != 0 || w->n % 16 != 0) {
    set_error("moe_fp4_grouped_gemm: %s needs k %% 128 == 0 and n %% 16 == 0 (n=%d k=%d)", name, w->n, w->k);
    return MOE_ERR_UNSUPPORTED;
  }
  if (w->format == MOE_FP4_MXC && w->k % 512 != 0) {
    set_error("moe_fp4_grouped_gemm: %s compact weights need k %% 512 == 0 (k=%d)", name, w->k);
    return MOE_ERR_UNSUPPORTED;
  }
  if (w->flags & MOE_FP4_TILED) {
    MOE_CHECK(w->k % 512 == 0, "moe_fp4_grouped_gemm: %s tiled layout needs k %% 512 == 0 (k=%d)", name, w->k);
    MOE_CHECK(aligned16(w->scale), "moe_fp4_grouped_gemm: %s tiled scales not 16-byte aligned", name);
  }
  return MOE_OK;
}

moe_status moe_fp4_grouped_gemm(const moe_act* a, const moe_fp4_weights* w0, const moe_fp4_weights* w1,
                                moe_epilogue epi, const int32_t* expert_offsets, int64_t rows, const moe_out* out,
                                int32_t algo, hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(a && out && expert_offsets, "moe_fp4_grouped_gemm: NULL argument");
  MOE_CHECK(epi == MOE_EPI_NONE || epi == MOE_EPI_SWIGLU, "moe_fp4_grouped_gemm: bad epilogue");
  moe_status st = check_weights(w0, "w0");
  if (st) return st;
  if (epi == MOE_EPI_SWIGLU) {
    st = check_weights(w1, "w1");
    if (st) return st;
    MOE_CHECK(w1->format == w0->format && w1->flags == w0->flags && w1->num_experts == w0->num_experts &&
                  w1->n == w0->n && w1->k == w0->k,
              "moe_fp4_grouped_gemm: w0 / w1 differ");
  }
  MOE_CHECK(rows >= 0, "moe_fp4_grouped_gemm: rows < 0");
  MOE_CHECK(a->mode >= MOE_ACT_BF16 && a->mode <= MOE_ACT_NVFP4_PLANES, "moe_fp4_grouped_gemm: bad activation mode");
  MOE_CHECK(a->data != nullptr && aligned16(a->data), "moe_fp4_grouped_gemm: activation data NULL or unaligned");
  const bool scaled = a->mode == MOE_ACT_MXFP8 || a->mode == MOE_ACT_NVFP4_PLANES;
  if (a->mode != MOE_ACT_BF16) MOE_CHECK(a->scales != nullptr, "moe_fp4_grouped_gemm: activations need scales");
  if (a->mode == MOE_ACT_NVFP4)
    MOE_CHECK(is_pow2_float(a->input_scale), "moe_fp4_grouped_gemm: input_scale must be a power of two");
  if (a->gather) MOE_CHECK(a->gather_div >= 1, "moe_fp4_grouped_gemm: gather_div < 1");
  MOE_CHECK(a->rows_src >= 0, "moe_fp4_grouped_gemm: rows_src < 0");
  // bytes per source row of the token operand
  const int64_t a_row_bytes = a->mode == MOE_ACT_BF16 ? (int64_t)w0->k * 2
                              : a->mode == MOE_ACT_NVFP4 ? (int64_t)w0->k / 2
                              : a->mode == MOE_ACT_MXFP8 ? (int64_t)w0->k : (int64_t)w0->k * 2;
  if (a->rows_src * a_row_bytes >= ((int64_t)1 << 31)) {
    set_error("moe_fp4_grouped_gemm: activations larger than 2 GiB are not supported");
    return MOE_ERR_UNSUPPORTED;
  }
  MOE_CHECK(out->data || out->codes || out->dequant, "moe_fp4_grouped_gemm: no output");
  MOE_CHECK(out->format >= MOE_OUT_NVFP4 && out->format <= MOE_OUT_NVFP4_PLANES, "moe_fp4_grouped_gemm: bad out.format");
  if (out->data) MOE_CHECK(aligned16(out->data), "moe_fp4_grouped_gemm: output not 16-byte aligned");
  if (out->dequant) {
    MOE_CHECK(aligned16(out->dequant), "moe_fp4_grouped_gemm: dequant output not 16-byte aligned");
    MOE_CHECK(out->format == MOE_OUT_NVFP4, "moe_fp4_grouped_gemm: dequant output is for the NVFP4 format");
  }
  if (out->codes) MOE_CHECK(out->scales != nullptr, "moe_fp4_grouped_gemm: quantised output needs scales");
  if (out->codes || out->dequant)
    MOE_CHECK(is_pow2_float(out->output_scale), "moe_fp4_grouped_gemm: output_scale must be a power of two");
  if (out->format != MOE_OUT_NVFP4) {
    MOE_CHECK(out->codes != nullptr, "moe_fp4_grouped_gemm: MXFP8 / plane output needs codes");
    MOE_CHECK(((uintptr_t)out->codes & 3) == 0, "moe_fp4_grouped_gemm: MXFP8 / plane codes not 4-byte aligned");
    if (out->format == MOE_OUT_MXFP8) MOE_CHECK(w0->n % 32 == 0, "moe_fp4_grouped_gemm: MXFP8 output needs n %% 32 == 0");
    int e;
    (void)frexpf(out->output_scale, &e);
    MOE_CHECK(e - 1 >= -100 && e - 1 <= 100, "moe_fp4_grouped_gemm: output_scale outside [2^-100, 2^100]");
    if (!scaled) {
      set_error("moe_fp4_grouped_gemm: MXFP8 / plane outputs come from the MXFP8 / plane activation modes");
      return MOE_ERR_UNSUPPORTED;
    }
  }
  MOE_CHECK(algo >= MOE_ALGO_AUTO && algo <= MOE_ALGO_PREFILL, "moe_fp4_grouped_gemm: bad algo");
  if (out->row_sumsq) {
    MOE_CHECK(epi == MOE_EPI_NONE, "moe_fp4_grouped_gemm: row_sumsq is for the down projection (MOE_EPI_NONE)");
    MOE_CHECK(((uintptr_t)out->row_sumsq & 3) == 0, "moe_fp4_grouped_gemm: row_sumsq not 4-byte aligned");
    // the sums come from the MFMA-tiled kernels' epilogue
    if (algo == MOE_ALGO_DECODE || w0->n % 256 != 0 || w0->k % 256 != 0 || w0->num_experts > 1000) {
      set_error("moe_fp4_grouped_gemm: row_sumsq needs the MFMA-tiled kernels (algo AUTO or PREFILL, n %% 256 == 0, "
                "k %% 256 == 0, <= 1000 experts)");
      return MOE_ERR_UNSUPPORTED;
    }
  }
  if (w0->format == MOE_FP4_MXC) {
    // the compact format is the weight-streaming kernel's (decode) storage
    if (scaled || out->row_sumsq || algo == MOE_ALGO_PREFILL) {
      set_error("moe_fp4_grouped_gemm: compact (MXC) weights run the weight-streaming kernel only: BF16 / NVFP4 "
                "activations, algo AUTO or DECODE, no row_sumsq");
      return MOE_ERR_UNSUPPORTED;
    }
  }
  if (scaled) {
    MOE_CHECK(w0->format == MOE_FP4_MX || (w0->flags & MOE_FP4_MX_EXACT),
              "moe_fp4_grouped_gemm: block-scaled MFMA modes need MX weights or NV weights flagged MX_EXACT");
      const int bn = epi == MOE_EPI_SWIGLU ? 256 : 512;
    if (w0->n % bn != 0 || w0->k % 256 != 0 || w0->num_experts > 1000) {
      set_error("moe_fp4_grouped_gemm: block-scaled MFMA modes need n %% %d == 0, k %% 256 == 0 and <= 1000 experts "
                "(n=%d k=%d E=%d)", bn, w0->n, w0->k, w0->num_experts);
      return MOE_ERR_UNSUPPORTED;
    }
  }
  if (rows == 0) return MOE_OK;

  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.a_data = (const uint8_t*)a->data;
  g.a_scales = a->scales;
  g.a_gscale = a->mode == MOE_ACT_NVFP4 ? a->input_scale : 1.0f;
  g.gather = a->gather;
  g.a_bytes = a->rows_src * a_row_bytes;
  g.gather_div = a->gather ? a->gather_div : 1;
  g.w_packed[0] = w0->packed;
  g.w_scale[0] = w0->scale;
  g.w_global[0] = w0->global_scale;
  const moe_fp4_weights* wl = epi == MOE_EPI_SWIGLU ? w1 : w0;
  g.w_packed[1] = wl->packed;
  g.w_scale[1] = wl->scale;
  g.w_global[1] = wl->global_scale;
  g.E = w0->num_experts;
  g.N = w0->n;
  g.K = w0->k;
  g.offsets = expert_offsets;
  g.rows = rows;
  g.out_bf16 = (uint16_t*)out->data;
  g.out_codes = out->codes;
  g.out_scales = out->scales;
  const bool nvfp4_out = out->codes || out->dequant;
  g.out_inv_g = nvfp4_out ? 1.0f / out->output_scale : 1.0f;
  g.out_dq = (uint16_t*)out->dequant;
  g.out_g = nvfp4_out ? out->output_scale : 1.0f;
  g.out_format = out->format;
  g.out_sumsq = out->row_sumsq;
  {
    int e;
    (void)frexpf(g.out_g, &e);
    g.out_g_log2 = e - 1;
  }
  g.tiled = (w0->flags & MOE_FP4_TILED) != 0;

  const bool swiglu = epi == MOE_EPI_SWIGLU;
  if (scaled) return launch_gemm_scaled(g, swiglu, a->mode == MOE_ACT_NVFP4_PLANES, w0->format == MOE_FP4_NV, stream);
  // weight scale format: 0 MXFP4, 1 NVFP4 with power-of-two scales, 2 NVFP4 with any scales, 3 compact MXFP4
  const int wf = w0->format == MOE_FP4_MX    ? 0
                 : w0->format == MOE_FP4_MXC ? 3
                                             : ((w0->flags & (MOE_FP4_SCALES_POW2 | MOE_FP4_MX_EXACT)) ? 1 : 2);
  const bool a_nv = a->mode == MOE_ACT_NVFP4;
  if (wf == 3) return launch_gemm_decode(g, swiglu, wf, a_nv, rows, stream);
  int use = algo;
  // measured crossover (decode weights, 256 experts): the MFMA-tiled kernels win
  // the layer from 4 rows per expert on average (1024 rows), the weight-streaming
  // kernel below it
  if (use == MOE_ALGO_AUTO) use = (rows >= 4LL * g.E || out->row_sumsq) ? MOE_ALGO_PREFILL : MOE_ALGO_DECODE;
  if (use == MOE_ALGO_PREFILL) return launch_gemm_prefill(g, swiglu, wf, a_nv, rows, stream);
  return launch_gemm_decode(g, swiglu, wf, a_nv, rows, stream);
}

moe_status moe_combine(const void* expert_out, const int32_t* slot_rows, const float* topk_weights,
                       const void* residual, int64_t T, int32_t top_k, int32_t h, void* y, hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(T >= 0 && top_k >= 1 && top_k <= 32, "moe_combine: bad T / top_k");
  MOE_CHECK(h >= 8 && h % 8 == 0, "moe_combine: h %% 8 != 0");
  if (T == 0) return MOE_OK;
  MOE_CHECK(expert_out && slot_rows && topk_weights && y, "moe_combine: NULL pointer");
  MOE_CHECK(aligned16(expert_out) && aligned16(y) && (!residual || aligned16(residual)),
            "moe_combine: bf16 buffers must be 16-byte aligned");
  return launch_combine(expert_out, slot_rows, topk_weights, residual, T, top_k, h, y, stream);
}

moe_status fp4_transcode_mx_to_nv(const uint8_t* mx_scale, const uint8_t* packed, int64_t num_mats, int32_t n,
                                  int32_t k, uint8_t* nv_scale, float* global_scale, int64_t* counters,
                                  hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(num_mats >= 0 && n >= 1 && k >= 32, "fp4_transcode_mx_to_nv: bad sizes");
  MOE_CHECK(k % 32 == 0 && n % 16 == 0, "fp4_transcode_mx_to_nv: needs k %% 32 == 0 and n %% 16 == 0");
  MOE_CHECK(counters != nullptr, "fp4_transcode_mx_to_nv: counters is NULL");
  if (num_mats > 0) {
    MOE_CHECK(mx_scale && packed && nv_scale && global_scale, "fp4_transcode_mx_to_nv: NULL pointer");
    MOE_CHECK(aligned16(mx_scale) && aligned16(packed) && aligned16(nv_scale),
              "fp4_transcode_mx_to_nv: buffers must be 16-byte aligned");
  }
  return launch_transcode(mx_scale, packed, num_mats, n, k, nv_scale, global_scale, counters, stream);
}

moe_status moe_fp4_compact_mx(const uint8_t* mx_scale, const uint8_t* packed, int64_t num_mats, int32_t n, int32_t k,
                              uint8_t* exp_codes, float* global_base, int64_t* counters, hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(num_mats >= 0 && n >= 16 && k >= 512, "moe_fp4_compact_mx: bad sizes");
  MOE_CHECK(k % 512 == 0 && n % 16 == 0, "moe_fp4_compact_mx: needs k %% 512 == 0 and n %% 16 == 0");
  MOE_CHECK(counters != nullptr && ((uintptr_t)counters & 7) == 0, "moe_fp4_compact_mx: counters NULL or unaligned");
  MOE_CHECK(num_mats * (int64_t)n * (k / 32) < ((int64_t)1 << 40), "moe_fp4_compact_mx: too many blocks");
  if (num_mats > 0) {
    MOE_CHECK(mx_scale && packed && exp_codes && global_base, "moe_fp4_compact_mx: NULL pointer");
    MOE_CHECK(aligned16(mx_scale) && aligned16(packed) && aligned16(exp_codes),
              "moe_fp4_compact_mx: buffers must be 16-byte aligned");
    MOE_CHECK(num_mats < ((int64_t)1 << 31), "moe_fp4_compact_mx: too many matrices");
  }
  return launch_compact(mx_scale, packed, num_mats, n, k, exp_codes, global_base, counters, stream);
}

moe_status moe_fp4_tile_weights(moe_fp4_format format, int32_t num_experts, int32_t n, int32_t k,
                                const uint8_t* packed, const uint8_t* scale, uint8_t* packed_tiled,
                                uint8_t* scale_tiled, hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(format == MOE_FP4_MX || format == MOE_FP4_NV || format == MOE_FP4_MXC, "moe_fp4_tile_weights: bad format");
  MOE_CHECK(num_experts >= 0 && n >= 16 && k >= 512, "moe_fp4_tile_weights: bad sizes");
  MOE_CHECK(n % 16 == 0 && k % 512 == 0, "moe_fp4_tile_weights: needs n %% 16 == 0 and k %% 512 == 0");
  if (num_experts == 0) return MOE_OK;
  MOE_CHECK(packed && scale && packed_tiled && scale_tiled, "moe_fp4_tile_weights: NULL pointer");
  MOE_CHECK(aligned16(packed) && aligned16(scale) && aligned16(packed_tiled) && aligned16(scale_tiled),
            "moe_fp4_tile_weights: buffers must be 16-byte aligned");
  const uint64_t cb = (uint64_t)num_experts * (uint64_t)n * (uint64_t)(k / 2);
  const uint64_t sb = (uint64_t)num_experts * (uint64_t)n *
                      (uint64_t)(format == MOE_FP4_NV ? k / 16 : format == MOE_FP4_MXC ? k / 64 : k / 32);
  auto overlap = [](const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  MOE_CHECK(!overlap(packed, cb, packed_tiled, cb) && !overlap(scale, sb, scale_tiled, sb) &&
                !overlap(packed, cb, scale_tiled, sb) && !overlap(scale, sb, packed_tiled, cb) &&
                !overlap(packed_tiled, cb, scale_tiled, sb),
            "moe_fp4_tile_weights: outputs overlap inputs or each other");
  return launch_tile(format == MOE_FP4_NV ? 1 : (format == MOE_FP4_MXC ? 2 : 0), num_experts, n, k, packed, scale,
                     packed_tiled, scale_tiled, stream);
}

moe_status moe_quantize_nvfp4(const void* x, int64_t rows, int32_t k, float input_scale, uint8_t* codes,
                              uint8_t* scales, void* dequant, hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(rows >= 0 && k >= 32 && k % 32 == 0, "moe_quantize_nvfp4: needs k %% 32 == 0");
  MOE_CHECK(is_pow2_float(input_scale), "moe_quantize_nvfp4: input_scale must be a power of two");
  if (rows == 0) return MOE_OK;
  MOE_CHECK(x && codes && scales, "moe_quantize_nvfp4: NULL pointer");
  MOE_CHECK(aligned16(x) && ((uintptr_t)codes & 7u) == 0, "moe_quantize_nvfp4: misaligned buffers");
  if (dequant) MOE_CHECK(aligned16(dequant), "moe_quantize_nvfp4: dequant output not 16-byte aligned");
  return launch_quant(x, rows, k, input_scale, codes, scales, dequant, stream);
}

moe_status moe_reap_saliency_accumulate(const float* row_sumsq, int64_t rows, int32_t parts,
                                        const int32_t* expert_offsets, int32_t num_experts,
                                        const int32_t* sorted_slots, const float* topk_weights, double* saliency_sum,
                                        int64_t* counts, hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(rows >= 0 && parts >= 1 && num_experts >= 0, "moe_reap_saliency_accumulate: bad sizes");
  if (rows == 0 || num_experts == 0) return MOE_OK;
  MOE_CHECK(row_sumsq && expert_offsets && sorted_slots && topk_weights && saliency_sum && counts,
            "moe_reap_saliency_accumulate: NULL pointer");
  MOE_CHECK(((uintptr_t)saliency_sum & 7) == 0 && ((uintptr_t)counts & 7) == 0,
            "moe_reap_saliency_accumulate: sums / counts not 8-byte aligned");
  return launch_saliency(row_sumsq, rows, parts, expert_offsets, num_experts, sorted_slots, topk_weights, saliency_sum,
                         counts, stream);
}

moe_status moe_quantize_mxfp8(const void* x, int64_t rows, int32_t k, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(rows >= 0 && k >= 32 && k % 32 == 0, "moe_quantize_mxfp8: needs k %% 32 == 0");
  if (rows == 0) return MOE_OK;
  MOE_CHECK(x && codes && scales, "moe_quantize_mxfp8: NULL pointer");
  MOE_CHECK(aligned16(x) && aligned16(codes), "moe_quantize_mxfp8: misaligned buffers");
  return launch_quant_mxfp8(x, rows, k, codes, scales, stream);
}

moe_status moe_quantize_nvfp4_planes(const void* x, int64_t rows, int32_t k, float input_scale, uint8_t* planes,
                                     uint8_t* plane_scales, hipStream_t stream) {
  g_err[0] = 0;
  MOE_CHECK(rows >= 0 && k >= 32 && k % 32 == 0, "moe_quantize_nvfp4_planes: needs k %% 32 == 0");
  MOE_CHECK(is_pow2_float(input_scale), "moe_quantize_nvfp4_planes: input_scale must be a power of two");
  int e;
  (void)frexpf(input_scale, &e);
  MOE_CHECK(e - 1 >= -100 && e - 1 <= 100, "moe_quantize_nvfp4_planes: input_scale outside [2^-100, 2^100]");
  if (rows == 0) return MOE_OK;
  MOE_CHECK(x && planes && plane_scales, "moe_quantize_nvfp4_planes: NULL pointer");
  MOE_CHECK(aligned16(x) && aligned16(planes), "moe_quantize_nvfp4_planes: misaligned buffers");
  return launch_quant_planes(x, rows, k, input_scale, planes, plane_scales, stream);
}

}  // extern "C"
