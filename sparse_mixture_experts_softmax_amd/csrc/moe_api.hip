// C ABI front end: argument validation, workspace layout and launch order.
// Every check runs on the host before anything is enqueued; nothing here
// allocates, frees or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

thread_local std::string g_last_error;
thread_local Prof g_prof;  // one-shot request from moe_profile_next_forward

// Scratch space of moe_forward_noalloc: one copy per GPU, placed in device memory when the code
// object is loaded there. In host code `scratch` names a host-side stand-in, never the device
// memory: host code uses only the per-device address hipGetSymbolAddress returns (g_scratch_at).
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_at[kMaxDevices] = {};

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_dims(const moe_dims* dm) {
  if (!dm) return fail(MOE_ERR_INVALID_ARG, "dims is NULL");
  if (dm->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld < 0", (long long)dm->T);
  if (dm->dtype != MOE_F32 && dm->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "dtype %d is neither MOE_F32 (0) nor MOE_BF16 (1)", dm->dtype);
  if (dm->renormalize != 0 && dm->renormalize != 1)
    return fail(MOE_ERR_INVALID_ARG, "renormalize must be 0 or 1, got %d", dm->renormalize);
  if (dm->E < 1) return fail(MOE_ERR_INVALID_ARG, "E = %d < 1", dm->E);
  if (dm->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 1024", dm->E);
  if (dm->k < 1 || dm->k > dm->E) return fail(MOE_ERR_INVALID_ARG, "k = %d outside [1, E = %d]", dm->k, dm->E);
  if (dm->k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k = %d > %d", dm->k, kMaxK);
  if (dm->d < 8 || dm->d % 8) return fail(MOE_ERR_INVALID_ARG, "d = %d is not a positive multiple of 8", dm->d);
  if (dm->I < 8 || dm->I % 8) return fail(MOE_ERR_INVALID_ARG, "I = %d is not a positive multiple of 8", dm->I);
  if (dm->I_shared < 0 || dm->I_shared % 8)
    return fail(MOE_ERR_INVALID_ARG, "I_shared = %d is not 0 or a positive multiple of 8", dm->I_shared);
  // T*k + T < 2^31, tested without forming the product (T may be near INT64_MAX)
  if (dm->T > ((1LL << 31) - 1) / (dm->k + 1))
    return fail(MOE_ERR_UNSUPPORTED, "T*k + T with T = %lld, k = %d does not fit in int32", (long long)dm->T, dm->k);
  return MOE_OK;
}

moe_status check_ptr(const void* p, size_t align, const char* name, bool required = true) {
  if (!p) return required ? fail(MOE_ERR_INVALID_ARG, "%s is NULL", name) : MOE_OK;
  if (!aligned(p, align)) return fail(MOE_ERR_INVALID_ARG, "%s = %p is not %zu-byte aligned", name, p, align);
  return MOE_OK;
}

#define MOE_TRY(expr)                   \
  do {                                  \
    moe_status _st = (expr);            \
    if (_st != MOE_OK) return _st;      \
  } while (0)

moe_status check_ws(const moe_dims& dm, const Layout& L, const void* ws, size_t ws_bytes) {
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
  if (!aligned(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace %p is not 256-byte aligned", ws);
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  (void)dm;
  return MOE_OK;
}

}  // namespace

Layout make_layout(const moe_dims& dm) {
  Layout L;
  const int64_t T = dm.T;
  const int64_t Tk = T * dm.k;
  const size_t esz = dm.dtype == MOE_F32 ? 4 : 2;
  // Router. bf16 x with enough tokens: MFMA on 128 x 256 or 128 x 512 tiles over K' = 3d (W_r
  // split into three bf16 parts). Otherwise fp32 vector ALUs on 64 x 64 tiles. Either way the K dimension
  // is split when the (token x expert) tiles alone would leave most of the 256 CUs idle.
  L.router_mfma = dm.dtype == MOE_BF16 && T >= 256 && dm.E % 256 == 0 && dm.d % 32 == 0 &&
                  (uint64_t)T * dm.d * 2 < (1ull << 32);
  int64_t splits, kchunk;
  L.router_wn = 2;
  if (L.router_mfma) {
    // 128 x 512 tiles (one workgroup per CU) where the experts divide them: the long K' = 3d
    // loop moves fewer L2 -> LDS bytes per FLOP than on 128 x 256 tiles
    L.router_wn = dm.E % 512 == 0 ? 4 : 2;
    const int64_t base_tiles = ((T + 127) / 128) * (dm.E / (128 * L.router_wn));
    const int64_t ksteps = 3 * (int64_t)dm.d / 32;
    // one workgroup per CU for few tiles (more splits only add partial sums for the top-k to
    // read); with 128 x 256 tiles two per CU (a second split) once the tiles alone cover half
    // the CUs
    const int64_t target = L.router_wn == 2 && base_tiles >= 128 ? 512 : 256;
    splits = (target + base_tiles - 1) / base_tiles;
    if (splits > 8) splits = 8;
    if (splits > ksteps / 8) splits = ksteps / 8 > 0 ? ksteps / 8 : 1;
    if (splits < 1) splits = 1;
    kchunk = (ksteps + splits - 1) / splits;
    splits = (ksteps + kchunk - 1) / kchunk;
  } else {
    const int64_t base_tiles = ((T + kRouterTileT - 1) / kRouterTileT) * ((dm.E + kRouterTileE - 1) / kRouterTileE);
    splits = base_tiles > 0 ? (512 + base_tiles - 1) / base_tiles : 1;
    const int64_t max_splits = dm.d / 256 > 0 ? dm.d / 256 : 1;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    kchunk = (dm.d + splits - 1) / splits;
    kchunk = (kchunk + kRouterKStep - 1) / kRouterKStep * kRouterKStep;
    splits = (dm.d + kchunk - 1) / kchunk;
  }
  L.router_splits = (int)splits;
  L.router_kchunk = (int)kchunk;
  L.nchunks = (T + kPermuteChunk - 1) / kPermuteChunk;
  // a handful of tokens: the top-k picks go straight from LDS into the dispatch (one launch and
  // one dependent global round trip fewer, on a path that is latency-bound)
  L.route_fused = !L.router_mfma && T >= 1 && T <= 4 && dm.E > 64;
  const int smallest_bm = kF32BM;
  L.max_tiles = Tk / smallest_bm + dm.E + T / smallest_bm + 2;
  L.ldh = dm.I > dm.I_shared ? dm.I : dm.I_shared;
  L.rows_total = Tk + (dm.I_shared > 0 ? T : 0);

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  L.router_planes = take(L.router_mfma ? (size_t)3 * dm.d * dm.E * 2 : 0);
  L.logits = take((size_t)splits * T * dm.E * 4);
  L.topk_idx = take((size_t)Tk * 4);
  L.topk_w = take((size_t)Tk * 4);
  L.topk_gap = take((size_t)T * 4);
  L.chunk_counts = take((size_t)L.nchunks * dm.E * 4);
  L.offsets = take((size_t)(dm.E + 2) * 4);
  L.sorted_token = take((size_t)Tk * 4);
  L.slot_of = take((size_t)Tk * 4);
  L.tile_group = take((size_t)L.max_tiles * 4);
  L.tile_m0 = take((size_t)L.max_tiles * 4);
  L.tile_count = take(4);
  L.H = take((size_t)L.rows_total * L.ldh * esz);
  L.Y = take((size_t)L.rows_total * dm.d * esz);
  const int64_t stat_chunks = (T + 63) / 64;  // router statistics: 64-token chunks
  L.probs = take((size_t)T * dm.E * 4);
  L.stat_p = take((size_t)stat_chunks * dm.E * 8);
  L.stat_c = take((size_t)stat_chunks * dm.E * 4);
  const FfnPlan P = ffn_plan(dm);
  size_t part = 0;
  if (P.s1 > 1) part = (size_t)P.s1 * L.rows_total * P.part_cols1 * 4;
  // (gate/up partial rows for at least 8 splits: the FP8 skinny product sizes its split by them)
  if (P.skinny) part = std::max(part, (size_t)std::max(P.ks1, 8) * L.rows_total * P.part_cols1 * 4);
  if (P.skinny && P.ks2 > 1) part = std::max(part, (size_t)P.ks2 * L.rows_total * P.part_cols2 * 4);
  L.ffn_part = take(part);
  // arrival counters of the skinny down product's K split (last-arriver sum), one per
  // (group, column block)
  // (at one or two tokens at least d / 128: the FP8 skinny down product's per-panel counters)
  int64_t per_tile = P.skinny ? std::max(P.cb1, P.cb2) : 0;
  if (T >= 1 && T <= kSkinnyMaxT) per_tile = std::max<int64_t>(per_tile, dm.d / 128);
  L.ffn_cnt_each = L.max_tiles * per_tile;
  L.ffn_cnt_per_tile = (int)per_tile;
  L.ffn_cnt = take((size_t)2 * L.ffn_cnt_each * 4);
  L.hnorm = take((size_t)T * dm.d * esz);
  L.total = off;
  return L;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_kernel_name(const moe_dims* dims, int32_t kernel, int32_t fp8) {
  if (check_dims(dims) != MOE_OK) return nullptr;
  const moe_dims& dm = *dims;
  if (fp8 && !fp8_shape_ok(dm)) return nullptr;
  const Layout L = make_layout(dm);
  switch (kernel) {
    case MOE_KERNEL_ROUTER:
      return L.router_mfma ? (L.router_wn == 4 ? "router_mfma_kernel<4>" : "router_mfma_kernel<2>")
             : dm.T <= 64  ? "router_small_kernel"
                           : "router_logits_kernel";
    case MOE_KERNEL_PERMUTE:
      if (L.route_fused) return "route_dispatch_kernel";
      return L.nchunks == 1 ? "permute_one_chunk_kernel" : "permute_count_kernel";
    case MOE_KERNEL_FFN_GATE_UP:
      return fp8 ? ffn_fp8_kernel_name(dm, true) : ffn_kernel_name(dm, true);
    case MOE_KERNEL_FFN_DOWN:
      return fp8 ? ffn_fp8_kernel_name(dm, false) : ffn_kernel_name(dm, false);
    case MOE_KERNEL_COMBINE:
      return "combine_kernel";
    default:
      return nullptr;
  }
}

moe_status moe_profile_next_forward(int32_t kernel, hipEvent_t start, hipEvent_t stop) {
  if (kernel == MOE_KERNEL_NONE) {
    g_prof = Prof();
    return MOE_OK;
  }
  if (kernel < MOE_KERNEL_ROUTER || kernel > MOE_KERNEL_COMBINE)
    return fail(MOE_ERR_INVALID_ARG, "unknown kernel id %d", kernel);
  if (!start || !stop) return fail(MOE_ERR_INVALID_ARG, "profile events must not be NULL");
  g_prof.kernel = kernel;
  g_prof.start = start;
  g_prof.stop = stop;
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_dims* dims, size_t* bytes) {
  MOE_TRY(check_dims(dims));
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = make_layout(*dims).total;
  return MOE_OK;
}

moe_status moe_router_topk(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                           int32_t* topk_idx, float* topk_w, float* topk_gap, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (dm.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(x, 16, "x"));
  MOE_TRY(check_ptr(w_router, 4, "w_router"));
  MOE_TRY(check_ptr(router_bias, 4, "router_bias", false));
  MOE_TRY(check_ptr(topk_idx, 4, "topk_idx"));
  MOE_TRY(check_ptr(topk_w, 4, "topk_w"));
  MOE_TRY(check_ptr(topk_gap, 4, "topk_gap", false));
  const Layout L = make_layout(dm);
  MOE_TRY(check_ws(dm, L, ws, ws_bytes));
  hipError_t e = launch_router(dm, L, x, w_router, router_bias, topk_idx, topk_w, topk_gap, (char*)ws, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_router_topk");
  return MOE_OK;
}

moe_status moe_router_topk_stats(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                                 int32_t* topk_idx, float* topk_w, float* topk_gap, int32_t* expert_counts,
                                 float* prob_mean, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  MOE_TRY(check_ptr(expert_counts, 4, "expert_counts"));
  MOE_TRY(check_ptr(prob_mean, 4, "prob_mean"));
  MOE_TRY(check_ptr(x, 16, "x", dm.T > 0));
  MOE_TRY(check_ptr(w_router, 4, "w_router", dm.T > 0));
  MOE_TRY(check_ptr(router_bias, 4, "router_bias", false));
  MOE_TRY(check_ptr(topk_idx, 4, "topk_idx", dm.T > 0));
  MOE_TRY(check_ptr(topk_w, 4, "topk_w", dm.T > 0));
  MOE_TRY(check_ptr(topk_gap, 4, "topk_gap", false));
  const Layout L = make_layout(dm);
  MOE_TRY(check_ws(dm, L, ws, ws_bytes));
  hipError_t e;
  if (dm.T > 0) {
    e = launch_router(dm, L, x, w_router, router_bias, topk_idx, topk_w, topk_gap, (char*)ws, stream,
                      (float*)((char*)ws + L.probs));
    if (e != hipSuccess) return hip_fail(e, "moe_router_topk_stats");
  }
  e = launch_router_stats(dm, L, topk_idx, (char*)ws, expert_counts, prob_mean, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_router_topk_stats");
  return MOE_OK;
}

moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, int32_t* expert_offsets, int32_t* sorted_token,
                       int32_t* slot_of, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (dm.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(topk_idx, 4, "topk_idx"));
  MOE_TRY(check_ptr(expert_offsets, 4, "expert_offsets"));
  MOE_TRY(check_ptr(sorted_token, 4, "sorted_token"));
  MOE_TRY(check_ptr(slot_of, 4, "slot_of"));
  const Layout L = make_layout(dm);
  MOE_TRY(check_ws(dm, L, ws, ws_bytes));
  hipError_t e = launch_permute(dm, L, topk_idx, expert_offsets, sorted_token, slot_of, (char*)ws, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_permute");
  return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_dims* dims, const void* x, const int32_t* expert_offsets,
                           const int32_t* sorted_token, const void* wg, const void* wu, const void* wd,
                           const void* wg_s, const void* wu_s, const void* wd_s, void* y, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (dm.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(x, 16, "x"));
  MOE_TRY(check_ptr(expert_offsets, 4, "expert_offsets"));
  MOE_TRY(check_ptr(sorted_token, 4, "sorted_token"));
  MOE_TRY(check_ptr(wg, 16, "wg"));
  MOE_TRY(check_ptr(wu, 16, "wu"));
  MOE_TRY(check_ptr(wd, 16, "wd"));
  const bool hs = dm.I_shared > 0;
  MOE_TRY(check_ptr(wg_s, 16, "wg_s", hs));
  MOE_TRY(check_ptr(wu_s, 16, "wu_s", hs));
  MOE_TRY(check_ptr(wd_s, 16, "wd_s", hs));
  MOE_TRY(check_ptr(y, 16, "y"));
  const Layout L = make_layout(dm);
  MOE_TRY(check_ws(dm, L, ws, ws_bytes));
  hipError_t e = launch_grouped_ffn(dm, L, x, expert_offsets, sorted_token, wg, wu, wd, wg_s, wu_s, wd_s, y,
                                    (char*)ws, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn");
  return MOE_OK;
}

moe_status moe_combine(const moe_dims* dims, const void* y, const int32_t* slot_of, const float* topk_w, void* out,
                       hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (dm.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(y, 16, "y"));
  MOE_TRY(check_ptr(slot_of, 4, "slot_of"));
  MOE_TRY(check_ptr(topk_w, 4, "topk_w"));
  MOE_TRY(check_ptr(out, 16, "out"));
  hipError_t e = launch_combine(dm, y, slot_of, topk_w, nullptr, out, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_combine");
  return MOE_OK;
}

moe_status moe_combine_residual(const moe_dims* dims, const void* y, const int32_t* slot_of, const float* topk_w,
                                const void* residual, void* out, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (dm.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(y, 16, "y"));
  MOE_TRY(check_ptr(slot_of, 4, "slot_of"));
  MOE_TRY(check_ptr(topk_w, 4, "topk_w"));
  MOE_TRY(check_ptr(residual, 16, "residual"));
  MOE_TRY(check_ptr(out, 16, "out"));
  hipError_t e = launch_combine(dm, y, slot_of, topk_w, residual, out, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_combine_residual");
  return MOE_OK;
}

moe_status moe_rmsnorm(const moe_dims* dims, const void* x, const void* gamma, double eps, void* h,
                       hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (!(eps >= 0.0 && eps < INFINITY)) return fail(MOE_ERR_INVALID_ARG, "eps = %g is not a finite value >= 0", eps);
  if (dm.T == 0) return MOE_OK;
  MOE_TRY(check_ptr(x, 16, "x"));
  MOE_TRY(check_ptr(gamma, 16, "gamma"));
  MOE_TRY(check_ptr(h, 16, "h"));
  hipError_t e = launch_rmsnorm(dm, x, gamma, eps, h, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_rmsnorm");
  return MOE_OK;
}

}  // extern "C"

namespace {

// The block on rows xin (the router and the experts see them); residual, when given, is added in
// the combine. Pointers validated by the caller.
moe_status forward_rows(const moe_dims& dm, const Layout& L, const void* xin, const void* residual,
                        const float* w_router, const float* router_bias, const void* wg, const void* wu,
                        const void* wd, const void* wg_s, const void* wu_s, const void* wd_s, void* out,
                        int32_t* topk_idx, float* topk_w, float* topk_gap, char* w, hipStream_t stream,
                        const Fp8Weights* fp8 = nullptr) {
  int32_t* idx = topk_idx ? topk_idx : (int32_t*)(w + L.topk_idx);
  float* tw = topk_w ? topk_w : (float*)(w + L.topk_w);
  int32_t* offsets = (int32_t*)(w + L.offsets);
  int32_t* sorted = (int32_t*)(w + L.sorted_token);
  int32_t* slot = (int32_t*)(w + L.slot_of);
  void* y = w + L.Y;
  const Prof prof = g_prof;
  g_prof = Prof();
  hipError_t e;
  if ((e = prof.begin(MOE_KERNEL_ROUTER, stream)) != hipSuccess) return hip_fail(e, "moe_forward/profile");
  if (L.route_fused)
    e = launch_router_logits(dm, L, xin, w_router, w, stream);
  else
    e = launch_router(dm, L, xin, w_router, router_bias, idx, tw, topk_gap, w, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/router");
  if ((e = prof.end(MOE_KERNEL_ROUTER, stream)) != hipSuccess) return hip_fail(e, "moe_forward/profile");
  if ((e = prof.begin(MOE_KERNEL_PERMUTE, stream)) != hipSuccess) return hip_fail(e, "moe_forward/profile");
  if (L.route_fused)
    e = launch_topk_dispatch(dm, L, router_bias, idx, tw, topk_gap, offsets, sorted, slot, w, stream, !fp8);
  else
    e = launch_permute(dm, L, idx, offsets, sorted, slot, w, stream, !fp8);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/permute");
  if ((e = prof.end(MOE_KERNEL_PERMUTE, stream)) != hipSuccess) return hip_fail(e, "moe_forward/profile");
  CombineFuse fuse{out, slot, tw, residual, false};
  if (fp8)
    e = launch_grouped_ffn_fp8(dm, L, xin, offsets, sorted, *fp8, y, w, stream, &prof, &fuse);
  else
    e = launch_grouped_ffn(dm, L, xin, offsets, sorted, wg, wu, wd, wg_s, wu_s, wd_s, y, w, stream, &prof, true,
                           &fuse);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/grouped_ffn");
  if ((e = prof.begin(MOE_KERNEL_COMBINE, stream)) != hipSuccess) return hip_fail(e, "moe_forward/profile");
  if (!fuse.done) e = launch_combine(dm, y, slot, tw, residual, out, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/combine");
  if ((e = prof.end(MOE_KERNEL_COMBINE, stream)) != hipSuccess) return hip_fail(e, "moe_forward/profile");
  return MOE_OK;
}

// Device address of the current device's scratch array, looked up on its first use there.
moe_status scratch_address(void** at) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "moe_forward_noalloc/hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: moe_forward_noalloc supports devices 0 .. %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_at[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "moe_forward_noalloc/hipGetSymbolAddress");
    if (!p || ((uintptr_t)p & 255u))
      return fail(MOE_ERR_HIP, "moe_forward_noalloc: scratch address %p is not 256-byte aligned", p);
    g_scratch_at[dev] = p;
  }
  *at = g_scratch_at[dev];
  return MOE_OK;
}

moe_status check_block_ptrs(const moe_dims& dm, const void* x, const float* w_router, const float* router_bias,
                            const void* wg, const void* wu, const void* wd, const void* wg_s, const void* wu_s,
                            const void* wd_s, const void* out, const int32_t* topk_idx, const float* topk_w,
                            const float* topk_gap) {
  MOE_TRY(check_ptr(x, 16, "x"));
  MOE_TRY(check_ptr(w_router, 4, "w_router"));
  MOE_TRY(check_ptr(router_bias, 4, "router_bias", false));
  MOE_TRY(check_ptr(wg, 16, "wg"));
  MOE_TRY(check_ptr(wu, 16, "wu"));
  MOE_TRY(check_ptr(wd, 16, "wd"));
  const bool hs = dm.I_shared > 0;
  MOE_TRY(check_ptr(wg_s, 16, "wg_s", hs));
  MOE_TRY(check_ptr(wu_s, 16, "wu_s", hs));
  MOE_TRY(check_ptr(wd_s, 16, "wd_s", hs));
  MOE_TRY(check_ptr(out, 16, "out"));
  MOE_TRY(check_ptr(topk_idx, 4, "topk_idx", false));
  MOE_TRY(check_ptr(topk_w, 4, "topk_w", false));
  MOE_TRY(check_ptr(topk_gap, 4, "topk_gap", false));
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                       const void* wg, const void* wu, const void* wd, const void* wg_s, const void* wu_s,
                       const void* wd_s, void* out, int32_t* topk_idx, float* topk_w, float* topk_gap, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (dm.T == 0) return MOE_OK;
  MOE_TRY(check_block_ptrs(dm, x, w_router, router_bias, wg, wu, wd, wg_s, wu_s, wd_s, out, topk_idx, topk_w,
                           topk_gap));
  const Layout L = make_layout(dm);
  MOE_TRY(check_ws(dm, L, ws, ws_bytes));
  return forward_rows(dm, L, x, nullptr, w_router, router_bias, wg, wu, wd, wg_s, wu_s, wd_s, out, topk_idx, topk_w,
                      topk_gap, (char*)ws, stream);
}

moe_status moe_forward_noalloc(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                               const void* wg, const void* wu, const void* wd, const void* wg_s, const void* wu_s,
                               const void* wd_s, void* out, int32_t* topk_idx, float* topk_w, float* topk_gap,
                               hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (dm.T == 0) return MOE_OK;
  MOE_TRY(check_block_ptrs(dm, x, w_router, router_bias, wg, wu, wd, wg_s, wu_s, wd_s, out, topk_idx, topk_w,
                           topk_gap));
  const Layout L = make_layout(dm);
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_forward_noalloc: these dims need %zu bytes of scratch, more than the %zu the library holds "
                "per GPU (use moe_forward with a workspace)",
                L.total, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  MOE_TRY(scratch_address(&ws));
  return forward_rows(dm, L, x, nullptr, w_router, router_bias, wg, wu, wd, wg_s, wu_s, wd_s, out, topk_idx, topk_w,
                      topk_gap, (char*)ws, stream);
}

moe_status moe_forward_fp8(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                           const uint8_t* wg, const uint8_t* wu, const uint8_t* wd, const float* sg, const float* su,
                           const float* sd, const uint8_t* wg_s, const uint8_t* wu_s, const uint8_t* wd_s,
                           const float* sg_s, const float* su_s, const float* sd_s, void* out, int32_t* topk_idx,
                           float* topk_w, float* topk_gap, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (!fp8_shape_ok(dm))
    return fail(MOE_ERR_UNSUPPORTED,
                "FP8 experts need bf16 activations, d %% 256 == 0, I and I_shared %% 128 == 0 (dtype %d, d %d, I %d, "
                "I_shared %d)",
                dm.dtype, dm.d, dm.I, dm.I_shared);
  if (dm.T == 0) return MOE_OK;
  const bool hs = dm.I_shared > 0;
  MOE_TRY(check_block_ptrs(dm, x, w_router, router_bias, wg, wu, wd, wg_s, wu_s, wd_s, out, topk_idx, topk_w,
                           topk_gap));
  MOE_TRY(check_ptr(sg, 4, "sg"));
  MOE_TRY(check_ptr(su, 4, "su"));
  MOE_TRY(check_ptr(sd, 4, "sd"));
  MOE_TRY(check_ptr(sg_s, 4, "sg_s", hs));
  MOE_TRY(check_ptr(su_s, 4, "su_s", hs));
  MOE_TRY(check_ptr(sd_s, 4, "sd_s", hs));
  const Layout L = make_layout(dm);
  MOE_TRY(check_ws(dm, L, ws, ws_bytes));
  const Fp8Weights W{wg, wu, wd, sg, su, sd, wg_s, wu_s, wd_s, sg_s, su_s, sd_s};
  return forward_rows(dm, L, x, nullptr, w_router, router_bias, wg, wu, wd, wg_s, wu_s, wd_s, out, topk_idx, topk_w,
                      topk_gap, (char*)ws, stream, &W);
}

moe_status moe_quantize_fp8(const void* w, int32_t dtype, int64_t batch, int32_t K, int32_t N, uint8_t* q,
                            float* scale, hipStream_t stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "dtype = %d", dtype);
  if (batch < 0 || K < 1 || N < 1 || batch > 65535)
    return fail(MOE_ERR_INVALID_ARG, "batch = %lld (0 .. 65535), K = %d, N = %d (>= 1)", (long long)batch, K, N);
  if (batch == 0) return MOE_OK;
  MOE_TRY(check_ptr(w, dtype == MOE_BF16 ? 2 : 4, "w"));
  MOE_TRY(check_ptr(q, 16, "q"));
  MOE_TRY(check_ptr(scale, 4, "scale"));
  if (K % 32 || N % 128)
    return fail(MOE_ERR_UNSUPPORTED, "FP8 code tiles need K %% 32 == 0 and N %% 128 == 0 (K = %d, N = %d)", K, N);
  hipError_t e = launch_quantize_fp8(w, dtype, batch, K, N, q, scale, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_quantize_fp8");
  return MOE_OK;
}

moe_status moe_forward_block(const moe_dims* dims, const void* x, const void* gamma, double eps,
                             const float* w_router, const float* router_bias, const void* wg, const void* wu,
                             const void* wd, const void* wg_s, const void* wu_s, const void* wd_s, void* out,
                             int32_t* topk_idx, float* topk_w, float* topk_gap, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& dm = *dims;
  if (!(eps >= 0.0 && eps < INFINITY)) return fail(MOE_ERR_INVALID_ARG, "eps = %g is not a finite value >= 0", eps);
  if (dm.T == 0) return MOE_OK;
  MOE_TRY(check_block_ptrs(dm, x, w_router, router_bias, wg, wu, wd, wg_s, wu_s, wd_s, out, topk_idx, topk_w,
                           topk_gap));
  MOE_TRY(check_ptr(gamma, 16, "gamma"));
  const Layout L = make_layout(dm);
  MOE_TRY(check_ws(dm, L, ws, ws_bytes));
  // the normalised rows have a workspace region of their own: the router and the gate/up product
  // read them, and no other step writes there
  char* w = (char*)ws;
  void* h = w + L.hnorm;
  hipError_t e = launch_rmsnorm(dm, x, gamma, eps, h, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_forward_block/rmsnorm");
  return forward_rows(dm, L, h, x, w_router, router_bias, wg, wu, wd, wg_s, wu_s, wd_s, out, topk_idx, topk_w,
                      topk_gap, w, stream);
}

}  // extern "C"
