// C ABI of the MoE layer (declared in include/moe.h): argument checks, workspace layout,
// and the launch sequence of the gfx950 kernels.  No device allocation, no host sync.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "kernels.h"
#include "moe.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Tile configuration from the expected rows per expert (host-known bounds only).
GemmKind choose_kind(long long rows_total, int groups, int cap) {
  const double mean = (double)rows_total / (double)groups;
  double mx = mean + 4.0 * sqrt(mean) + 2.0;
  if (cap >= 0) mx = std::min(mx, (double)cap);
  if (mx <= 16.0) return kGemmDecode;
  if (mean >= 384.0) return kGemmLarge;
  return kGemmStream;
}

// K chunks of the routed down product.  At decode sizes each expert has one m-tile, so the
// product has only E * d / 32 output tiles, each a long run of d_e / 64 K steps.  With 4-bit
// weights a decode tile takes so little LDS that several times more blocks fit on a CU than
// there are tiles; cutting K in two doubles the blocks streaming weights at once.  (With
// 8- and 16-bit weights the tiles already fill the CUs, and the extra partial sums only cost
// time.)  The combine sums the chunks' partial outputs.
int down_ksplit(const moe_shape& s, GemmKind kind) {
  if (kind != kGemmDecode || s.wfmt != MOE_W_MXFP4 || s.afmt != MOE_A_NATIVE) return 1;
  return s.d_e % 128 == 0 && s.d_e / 128 >= 16 ? 2 : 1;
}

struct Layout {
  size_t p_part, hist, chunk_base, counts, kept, offsets, row_token, row_of, tstart1, tstart2, logits;
  size_t x_perm, xq, h, o, sh_h, sh_o, tctr, total;
  int ksplit;   // K chunks of the routed down product in the forward (partials at o + c * T*k*d)
};

size_t elem_size(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

Layout layout(const moe_shape& s) {
  Layout L{};
  const size_t es = elem_size(s.dtype);
  const size_t nb = (size_t)route_blocks(s.T);
  const size_t E = (size_t)s.E, R = (size_t)s.T * (size_t)s.k;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align_up(bytes); return at; };
  L.p_part = take(nb * E * sizeof(float));
  L.hist = take(nb * E * sizeof(int32_t));
  L.chunk_base = take(nb * E * sizeof(int32_t));
  L.counts = take(E * sizeof(int32_t));
  L.kept = take(E * sizeof(int32_t));
  L.offsets = take((E + 1) * sizeof(int32_t));
  L.row_token = take(R * sizeof(int32_t));
  L.row_of = take(R * sizeof(int32_t));
  L.tstart1 = take((E + 1) * sizeof(int32_t));
  L.tstart2 = take((E + 1) * sizeof(int32_t));
  L.logits = take(router_logits_bytes(s.T, s.d, s.E));
  L.x_perm = take(R * (size_t)s.d * es);
  // MXFP8 activations: x (or x_perm) as codes [R, d] then scales [R, d/32]; h and the shared
  // expert's h as codes then scales inside their bf16-sized pieces (1 + 1/32 <= 2 bytes each)
  L.xq = take(s.afmt == MOE_A_MXFP8 ? R * (size_t)s.d + R * (size_t)(s.d / 32) : 0);
  L.h = take(R * (size_t)s.d_e * es);
  L.ksplit = down_ksplit(s, choose_kind(std::max<long long>((long long)R, 1), s.E, s.capacity));
  L.o = take(R * (size_t)s.d * sizeof(float) * (size_t)L.ksplit);
  L.sh_h = take((size_t)s.T * (size_t)s.d_e_shared * es);
  L.sh_o = take(s.d_e_shared > 0 ? (size_t)s.T * (size_t)s.d * sizeof(float) : 0);
  L.tctr = take(kTileCtrInts * sizeof(int32_t));   // work counters of the routed down product
  L.total = off;
  return L;
}

// Workspace of moe_backward.  Transposed operands of the weight-gradient products hold each
// expert's rows from a 64-aligned column (ldt bounds the padded total).
struct BwdLayout {
  size_t poff, koff_dense, ts1, ts2, g_row, wdT, wguT, dyb, a, b, hT, dab, dabT, part, dr, dX, xT, doT;
  size_t swdT, swguT, sa, sb, shT, sdab, sdabT, sdX, sdyT, sxT, dwr_part, logits, tctr, total;
  int ldt, ldts, npart;
  GemmKind kind, skind;
};

BwdLayout bwd_layout(const moe_shape& s) {
  BwdLayout L{};
  const size_t es = elem_size(s.dtype);
  const size_t E = (size_t)s.E, R = (size_t)s.T * (size_t)s.k, d = (size_t)s.d, de = (size_t)s.d_e;
  const size_t des = (size_t)s.d_e_shared, T = (size_t)s.T;
  L.kind = choose_kind(std::max<long long>((long long)R, 1), s.E, s.capacity);
  L.skind = choose_kind(std::max<long long>((long long)T, 1), 1, -1);
  L.ldt = (int)((R + 63 * E + 63) / 64 * 64);
  L.ldts = (int)((T + 63) / 64 * 64);
  L.npart = s.d_e / gemm_dgrad_part_cols(L.kind, s.d_e);
  const size_t ldt = (size_t)L.ldt, ldts = (size_t)L.ldts;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align_up(bytes); return at; };
  L.poff = take((E + 1) * sizeof(int32_t));
  L.koff_dense = take(2 * sizeof(int32_t));
  L.ts1 = take((E + 1) * sizeof(int32_t));
  L.ts2 = take((E + 1) * sizeof(int32_t));
  L.g_row = take(R * sizeof(float));
  L.wdT = take(E * de * d * es);
  L.wguT = take(E * d * 2 * de * es);
  L.dyb = take(s.dtype == MOE_BF16 ? T * d * es : 0);
  L.a = take(R * de * sizeof(float));
  L.b = take(R * de * sizeof(float));
  L.hT = take(de * ldt * es);
  L.dab = take(R * 2 * de * es);
  L.dabT = take(2 * de * ldt * es);
  L.part = take(R * (size_t)L.npart * sizeof(float));
  L.dr = take(T * E * sizeof(float));
  L.dX = take(R * d * sizeof(float));
  L.xT = take(d * ldt * es);
  L.doT = take(d * ldt * es);
  L.swdT = take(des * d * es);
  L.swguT = take(d * 2 * des * es);
  L.sa = take(T * des * sizeof(float));
  L.sb = take(T * des * sizeof(float));
  L.shT = take(des * ldts * es);
  L.sdab = take(T * 2 * des * es);
  L.sdabT = take(2 * des * ldts * es);
  L.sdX = take(des > 0 ? T * d * sizeof(float) : 0);
  L.sdyT = take(des > 0 ? d * ldts * es : 0);
  L.sxT = take(des > 0 ? d * ldts * es : 0);
  L.dwr_part = take(dwr_workspace_bytes(s.T, s.d, s.E));
  L.logits = take(router_logits_bytes(s.T, s.d, s.E));
  L.tctr = take(kTileCtrInts * sizeof(int32_t));   // work counters of the routed dX product
  L.total = off;
  return L;
}

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_NULL;
  if (s->T < 0 || s->d < 1 || s->d_e < 1 || s->E < 1 || s->k < 1 || s->k > s->E || s->d_e_shared < 0)
    return MOE_ERR_SHAPE;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->scoring != MOE_SCORE_SOFTMAX && s->scoring != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (s->n_group < 1 || s->topk_group < 1 || s->topk_group > s->n_group || s->E % s->n_group != 0)
    return MOE_ERR_SHAPE;
  if ((long long)s->k > (long long)s->topk_group * (s->E / s->n_group)) return MOE_ERR_SHAPE;
  if (s->wfmt != MOE_W_NATIVE && s->wfmt != MOE_W_FP8_E4M3 && s->wfmt != MOE_W_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (s->wfmt != MOE_W_NATIVE && s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->afmt != MOE_A_NATIVE && s->afmt != MOE_A_MXFP8) return MOE_ERR_UNSUPPORTED;
  if (s->afmt == MOE_A_MXFP8 && s->wfmt == MOE_W_NATIVE) return MOE_ERR_UNSUPPORTED;
  if (s->n_group > 64) return MOE_ERR_UNSUPPORTED;
  if (s->E > 1024 || s->k > 16) return MOE_ERR_UNSUPPORTED;
  if (s->d % 128 || s->d_e % 128 || s->d_e_shared % 128) return MOE_ERR_UNSUPPORTED;
  if ((long long)s->T * s->k >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  // the forward gathers rows of x with 32-bit byte offsets: T*d*elem_size < 2^32
  if ((long long)s->T * s->d * (s->dtype == MOE_BF16 ? 2 : 4) >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  // the gather addresses x_perm in 16-byte units with int32: T*k*d*elem_size / 16 < 2^31
  if ((long long)s->T * s->k * (long long)s->d * (s->dtype == MOE_BF16 ? 2 : 4) >= (1LL << 35))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Rows per tile of the gate/up (gated) or down product for this shape's formats.
int block_m(const moe_shape& s, GemmKind kind, bool gated) {
  return s.afmt == MOE_A_MXFP8 ? gemm_block_m_mx(kind) : gemm_block_m(kind, s.dtype, gated, s.wfmt);
}

// Upper bound on the number of m-tiles over all groups.
int max_m_tiles(long long rows_bound, int groups, int cap, int bm) {
  long long a = (rows_bound + bm - 1) / bm + groups;
  if (cap >= 0) {
    long long per = (std::min<long long>(cap, rows_bound) + bm - 1) / bm;
    a = std::min(a, per * groups);
  }
  return (int)std::min<long long>(a, 1LL << 30);
}

#define MOE_HIP(call)                               \
  do {                                              \
    if ((call) != hipSuccess) return MOE_ERR_HIP;   \
  } while (0)

template <typename P>
P* at(void* ws, size_t off) { return (P*)((char*)ws + off); }

moe_status run_router(const moe_shape& s, const void* x, const void* w_r, const float* b_r, int32_t* idx,
                      float* gate, int32_t* counts, float* f, float* P, float* aux, int32_t* kept,
                      int32_t* offsets, int bm1, int bm2, void* ws, hipStream_t st) {
  const Layout L = layout(s);
  const int nb = route_blocks(s.T);
  if (s.T > 0)
    MOE_HIP(launch_router(s.dtype, x, w_r, b_r, s.T, s.d, s.E, s.k, s.renormalize, s.scoring, s.n_group,
                          s.topk_group, idx, gate, at<float>(ws, L.p_part), at<int32_t>(ws, L.hist),
                          at<float>(ws, L.logits), st));
  MOE_HIP(launch_scan(at<int32_t>(ws, L.hist), at<float>(ws, L.p_part), nb, s.T, s.k, s.E, s.capacity, counts,
                      kept, offsets, at<int32_t>(ws, L.chunk_base), f, P, aux, bm1, at<int32_t>(ws, L.tstart1),
                      bm2, at<int32_t>(ws, L.tstart2), st));
  return MOE_OK;
}

// Row scales of FP8 weights, or all-NULL for native weights.
const moe_wscales kNoScales = {nullptr, nullptr, nullptr};

bool scales_ok(const moe_shape& s, const moe_wscales* sc) {
  return s.wfmt == MOE_W_NATIVE || (sc && sc->gate && sc->up && sc->down);
}

// The two products of the MXFP8-activation mode: A = MXFP8 rows (codes aq, scales as, row
// a_rows[r] when given), h as MXFP8 in the piece at h (codes [rows, d_e] then scales).
moe_status run_ffn_mx(const moe_shape& s, int G, const uint8_t* aq, const uint8_t* as, const int32_t* a_rows,
                      const int32_t* offsets, const int32_t* tstart1, const int32_t* tstart2, GemmKind kind,
                      int tiles1, int tiles2, int dense_rows, long long h_rows, int d_e, const void* wg,
                      const void* wu, const void* wd, const moe_wscales& sc, void* h, float* o, hipStream_t st) {
  uint8_t* hq = (uint8_t*)h;
  uint8_t* hs = hq + (size_t)h_rows * (size_t)d_e;
  MOE_HIP(launch_gemm_gateup_mx(kind, s.wfmt, aq, as, a_rows, wg, wu, sc.gate, sc.up, offsets, tstart1, G, dense_rows,
                                tiles1, d_e, s.d, hq, hs, st));
  MOE_HIP(launch_gemm_down_mx(kind, s.wfmt, hq, hs, wd, sc.down, offsets, tstart2, G, dense_rows, tiles2, s.d, d_e, o,
                              st));
  return MOE_OK;
}

moe_status run_ffn(const moe_shape& s, int G, const void* A, const int32_t* offsets, const int32_t* tstart1,
                   const int32_t* tstart2, GemmKind kind, int tiles1, int tiles2, int dense_rows, int d_e,
                   const void* wg, const void* wu, const void* wd, const moe_wscales& sc, void* h, float* o,
                   hipStream_t st) {
  MOE_HIP(launch_gemm_gateup(kind, s.dtype, s.wfmt, A, nullptr, wg, wu, (const float*)sc.gate, (const float*)sc.up,
                             offsets, tstart1, G, dense_rows, tiles1, d_e, s.d, h, st));
  MOE_HIP(launch_gemm_down(kind, s.dtype, s.wfmt, h, wd, (const float*)sc.down, offsets, tstart2, G, dense_rows,
                           tiles2, s.d, d_e, o, 1, 0, st));
  return MOE_OK;
}

// Host checks of moe_forward's arguments other than the workspace (shape, then pointers).
moe_status forward_args(const moe_shape* shape, const void* x, const void* w_r, const void* w_gate, const void* w_up,
                        const void* w_down, const void* ws_gate, const void* ws_up, const void* ws_down,
                        const moe_wscales* scales, const moe_wscales* shared_scales, const float* y,
                        const int32_t* idx, const float* gate, const int32_t* counts, const int32_t* kept,
                        const float* f, const float* P, const float* aux) {
  moe_status v = check_shape(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if ((s.T > 0 && (!x || !w_r || !w_gate || !w_up || !w_down || !y || !idx || !gate)) || !counts || !kept || !f ||
      !P || !aux)
    return MOE_ERR_NULL;
  if (s.d_e_shared > 0 && s.T > 0 && (!ws_gate || !ws_up || !ws_down)) return MOE_ERR_NULL;
  if (s.T > 0 && (!scales_ok(s, scales) || (s.d_e_shared > 0 && !scales_ok(s, shared_scales)))) return MOE_ERR_NULL;
  return MOE_OK;
}

// Scratch of moe_forward_noalloc: one copy per GPU (the code object's device memory), held
// until the process ends.  In host code `scratch` names a host-side stand-in, not the device
// memory: the device address comes from hipGetSymbolAddress, looked up once per device with
// that device current, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the device's first call).
moe_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: inconsistent or negative size";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or dtype outside the supported set";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP call failed";
  }
  return "unknown moe_status";
}

moe_status moe_capacity(int32_t T, int32_t k, int32_t E, double C, int32_t* cap) {
  if (!cap) return MOE_ERR_NULL;
  if (T < 0 || k < 1 || E < 1 || !(C >= 0.0) || !isfinite(C)) return MOE_ERR_SHAPE;
  const double v = floor(C * (double)T * (double)k / (double)E);
  if (v >= 2147483648.0) return MOE_ERR_SHAPE;
  *cap = (int32_t)v;
  return MOE_OK;
}

moe_status moe_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  *bytes = layout(*shape).total;
  return MOE_OK;
}

moe_status moe_route(const moe_shape* shape, const void* x, const void* w_r, const float* b_r, int32_t* idx,
                     float* gate, int32_t* counts, float* f, float* P, float* aux, void* ws, size_t ws_bytes,
                     void* stream) {
  moe_status v = check_shape(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if ((s.T > 0 && (!x || !w_r || !idx || !gate)) || !counts || !f || !P || !aux || !ws) return MOE_ERR_NULL;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return run_router(s, x, w_r, b_r, idx, gate, counts, f, P, aux, at<int32_t>(ws, L.kept),
                    at<int32_t>(ws, L.offsets), 1, 1, ws, (hipStream_t)stream);
}

moe_status moe_permute(const moe_shape* shape, const void* x, const int32_t* idx, int32_t* kept, int32_t* offsets,
                       int32_t* row_token, int32_t* row_of, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  moe_status v = check_shape(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if ((s.T > 0 && (!x || !idx || !row_token || !row_of || !x_perm)) || !kept || !offsets || !ws) return MOE_ERR_NULL;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int nb = route_blocks(s.T);
  if (s.T > 0) MOE_HIP(launch_hist(idx, s.T, s.k, s.E, at<int32_t>(ws, L.hist), st));
  MOE_HIP(launch_scan(at<int32_t>(ws, L.hist), nullptr, nb, s.T, s.k, s.E, s.capacity, nullptr, kept, offsets,
                      at<int32_t>(ws, L.chunk_base), nullptr, nullptr, nullptr, 1, at<int32_t>(ws, L.tstart1), 1,
                      at<int32_t>(ws, L.tstart2), st));
  if (s.T > 0)
    MOE_HIP(launch_rank_gather(s.dtype, x, idx, s.T, s.d, s.k, s.E, s.capacity, at<int32_t>(ws, L.chunk_base),
                               offsets, row_token, row_of, x_perm, st));
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_shape* shape, const void* x_perm, const int32_t* offsets, const void* w_gate,
                          const void* w_up, const void* w_down, const moe_wscales* scales, float* o, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status v = check_shape(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (!x_perm || !offsets || !w_gate || !w_up || !w_down || !o || !ws) return MOE_ERR_NULL;
  if (!scales_ok(s, scales)) return MOE_ERR_NULL;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const long long R = (long long)s.T * s.k;
  if (R == 0) return MOE_OK;
  const GemmKind kind = choose_kind(R, s.E, s.capacity);
  const int bm1 = block_m(s, kind, true), bm2 = block_m(s, kind, false);
  int32_t* ts1 = at<int32_t>(ws, L.tstart1);
  int32_t* ts2 = at<int32_t>(ws, L.tstart2);
  MOE_HIP(launch_tile_sched(offsets, s.E, bm1, ts1, bm2, ts2, st));
  if (s.afmt == MOE_A_MXFP8) {
    // every row of x_perm is quantised (rows past offsets[E] are unspecified and never read)
    uint8_t* xq = at<uint8_t>(ws, L.xq);
    uint8_t* xs = xq + (size_t)R * s.d;
    MOE_HIP(launch_mxfp8_quantize(x_perm, (int)R, s.d, xq, xs, st));
    return run_ffn_mx(s, s.E, xq, xs, nullptr, offsets, ts1, ts2, kind, max_m_tiles(R, s.E, -1, bm1),
                      max_m_tiles(R, s.E, -1, bm2), 0, R, s.d_e, w_gate, w_up, w_down, *scales, at<void>(ws, L.h), o,
                      st);
  }
  return run_ffn(s, s.E, x_perm, offsets, ts1, ts2, kind, max_m_tiles(R, s.E, -1, bm1), max_m_tiles(R, s.E, -1, bm2),
                 0, s.d_e, w_gate, w_up, w_down, s.wfmt != MOE_W_NATIVE ? *scales : kNoScales, at<void>(ws, L.h), o,
                 st);
}

moe_status moe_combine(const moe_shape* shape, const float* o, const int32_t* row_of, const float* gate,
                       const float* shared_out, float* y, void* stream) {
  moe_status v = check_shape(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if (!o || !row_of || !gate || !y) return MOE_ERR_NULL;
  MOE_HIP(launch_combine(o, row_of, gate, shared_out, y, s.T, s.d, s.k, 1, 0, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_forward(const moe_shape* shape, const void* x, const void* w_r, const float* b_r, const void* w_gate,
                       const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                       const void* ws_down, const moe_wscales* scales, const moe_wscales* shared_scales, float* y,
                       int32_t* idx, float* gate, int32_t* counts, int32_t* kept,
                       float* f, float* P, float* aux, int32_t* offsets, int32_t* row_token, int32_t* row_of,
                       void* ws, size_t ws_bytes, void* stream, void* const* stage_events) {
  moe_status v = forward_args(shape, x, w_r, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, scales, shared_scales, y,
                              idx, gate, counts, kept, f, P, aux);
  if (v != MOE_OK) return v;
  if (!ws) return MOE_ERR_NULL;
  const moe_shape& s = *shape;
  const bool w8 = s.wfmt != MOE_W_NATIVE;
  const moe_wscales& sc = w8 && s.T > 0 ? *scales : kNoScales;
  const moe_wscales& ssc = w8 && s.T > 0 && s.d_e_shared > 0 ? *shared_scales : kNoScales;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (!offsets) offsets = at<int32_t>(ws, L.offsets);
  if (!row_token) row_token = at<int32_t>(ws, L.row_token);
  if (!row_of) row_of = at<int32_t>(ws, L.row_of);
  // stage boundary marks (timing only)
  int next_stage = 0;
  auto mark = [&](int upto) -> bool {
    if (!stage_events) return true;
    for (; next_stage <= upto; ++next_stage)
      if (stage_events[next_stage] && hipEventRecord((hipEvent_t)stage_events[next_stage], st) != hipSuccess)
        return false;
    return true;
  };
#define MOE_MARK(i) \
  if (!mark(i)) return MOE_ERR_HIP

  const long long R = (long long)s.T * s.k;
  const GemmKind kind = choose_kind(std::max<long long>(R, 1), s.E, s.capacity);
  const int bm1 = block_m(s, kind, true), bm2 = block_m(s, kind, false);
  const int nb = route_blocks(s.T);
  int32_t* ts1 = at<int32_t>(ws, L.tstart1);
  int32_t* ts2 = at<int32_t>(ws, L.tstart2);
  MOE_MARK(MOE_STAGE_ROUTER);
  // A batch of one router block with few experts (decode) routes and dispatches in one launch;
  // its scan and permute stages are then empty.
  const bool small = route_small_ok(s.T, s.E);
  if (small) {
    SmallDispatch sd;
    sd.cap = s.capacity;
    sd.counts = counts;
    sd.kept = kept;
    sd.offsets = offsets;
    sd.f = f;
    sd.P = P;
    sd.aux = aux;
    sd.bm1 = bm1;
    sd.bm2 = bm2;
    sd.tstart1 = ts1;
    sd.tstart2 = ts2;
    sd.row_token = row_token;
    sd.row_of = row_of;
    MOE_HIP(launch_route_small(s.dtype, x, w_r, b_r, s.T, s.d, s.E, s.k, s.renormalize, s.scoring, s.n_group,
                               s.topk_group, idx, gate, sd, st));
  } else if (s.T > 0) {
    MOE_HIP(launch_router(s.dtype, x, w_r, b_r, s.T, s.d, s.E, s.k, s.renormalize, s.scoring, s.n_group,
                          s.topk_group, idx, gate, at<float>(ws, L.p_part), at<int32_t>(ws, L.hist),
                          at<float>(ws, L.logits), st));
  }
  MOE_MARK(MOE_STAGE_SCAN);
  if (!small)
    MOE_HIP(launch_scan(at<int32_t>(ws, L.hist), at<float>(ws, L.p_part), nb, s.T, s.k, s.E, s.capacity, counts,
                        kept, offsets, at<int32_t>(ws, L.chunk_base), f, P, aux, bm1, ts1, bm2, ts2, st));
  // The forward pass does not materialise x_perm: the permute stage produces the row
  // indices and the gate/up GEMM gathers token rows of x through them as it loads.
  MOE_MARK(MOE_STAGE_PERMUTE);
  if (!small && s.T > 0)
    MOE_HIP(launch_rank_gather(s.dtype, x, idx, s.T, s.d, s.k, s.E, s.capacity, at<int32_t>(ws, L.chunk_base),
                               offsets, row_token, row_of, nullptr, st));
  MOE_MARK(MOE_STAGE_GATE_UP);
  // MXFP8 activations: x is quantised once (per token row) for the routed and shared products
  uint8_t* xq = at<uint8_t>(ws, L.xq);
  uint8_t* xs = xq + (size_t)R * s.d;
  if (s.afmt == MOE_A_MXFP8 && s.T > 0) {
    MOE_HIP(launch_mxfp8_quantize(x, s.T, s.d, xq, xs, st));
    MOE_HIP(launch_gemm_gateup_mx(kind, s.wfmt, xq, xs, row_token, w_gate, w_up, sc.gate, sc.up, offsets, ts1, s.E, 0,
                                  max_m_tiles(R, s.E, s.capacity, bm1), s.d_e, s.d, at<uint8_t>(ws, L.h),
                                  at<uint8_t>(ws, L.h) + (size_t)R * s.d_e, st));
    MOE_MARK(MOE_STAGE_DOWN);
    MOE_HIP(launch_gemm_down_mx(kind, s.wfmt, at<uint8_t>(ws, L.h), at<uint8_t>(ws, L.h) + (size_t)R * s.d_e, w_down,
                                sc.down, offsets, ts2, s.E, 0, max_m_tiles(R, s.E, s.capacity, bm2), s.d, s.d_e,
                                at<float>(ws, L.o), st));
  } else if (s.T > 0) {
    MOE_HIP(launch_gemm_gateup(kind, s.dtype, s.wfmt, x, row_token, w_gate, w_up, (const float*)sc.gate,
                               (const float*)sc.up, offsets, ts1, s.E, 0, max_m_tiles(R, s.E, s.capacity, bm1), s.d_e,
                               s.d, at<void>(ws, L.h), st));
    MOE_MARK(MOE_STAGE_DOWN);
    MOE_HIP(launch_gemm_down(kind, s.dtype, s.wfmt, at<void>(ws, L.h), w_down, (const float*)sc.down, offsets, ts2, s.E, 0,
                             max_m_tiles(R, s.E, s.capacity, bm2), s.d, s.d_e, at<float>(ws, L.o), L.ksplit,
                             (size_t)R * s.d, st, at<int32_t>(ws, L.tctr)));
  }
  MOE_MARK(MOE_STAGE_SHARED_GATE_UP);
  const float* shared_out = nullptr;
  if (s.d_e_shared > 0 && s.T > 0 && s.afmt == MOE_A_MXFP8) {
    const GemmKind sk = choose_kind(s.T, 1, -1);
    const int sbm = gemm_block_m_mx(sk);
    uint8_t* shq = at<uint8_t>(ws, L.sh_h);
    MOE_HIP(launch_gemm_gateup_mx(sk, s.wfmt, xq, xs, nullptr, ws_gate, ws_up, ssc.gate, ssc.up, nullptr, nullptr, 1,
                                  s.T, (s.T + sbm - 1) / sbm, s.d_e_shared, s.d, shq,
                                  shq + (size_t)s.T * s.d_e_shared, st));
    MOE_MARK(MOE_STAGE_SHARED_DOWN);
    MOE_HIP(launch_gemm_down_mx(sk, s.wfmt, shq, shq + (size_t)s.T * s.d_e_shared, ws_down, ssc.down, nullptr,
                                nullptr, 1, s.T, (s.T + sbm - 1) / sbm, s.d, s.d_e_shared, at<float>(ws, L.sh_o), st));
    shared_out = at<float>(ws, L.sh_o);
  } else if (s.d_e_shared > 0 && s.T > 0) {
    const GemmKind sk = choose_kind(s.T, 1, -1);
    const int sbm1 = gemm_block_m(sk, s.dtype, true, s.wfmt), sbm2 = gemm_block_m(sk, s.dtype, false, s.wfmt);
    MOE_HIP(launch_gemm_gateup(sk, s.dtype, s.wfmt, x, nullptr, ws_gate, ws_up, (const float*)ssc.gate,
                               (const float*)ssc.up, nullptr, nullptr, 1,
                               s.T, (s.T + sbm1 - 1) / sbm1, s.d_e_shared, s.d, at<void>(ws, L.sh_h), st));
    MOE_MARK(MOE_STAGE_SHARED_DOWN);
    MOE_HIP(launch_gemm_down(sk, s.dtype, s.wfmt, at<void>(ws, L.sh_h), ws_down, (const float*)ssc.down, nullptr,
                             nullptr, 1, s.T,
                             (s.T + sbm2 - 1) / sbm2, s.d, s.d_e_shared, at<float>(ws, L.sh_o), 1, 0, st));
    shared_out = at<float>(ws, L.sh_o);
  }
  MOE_MARK(MOE_STAGE_COMBINE);
  if (s.T > 0)
    MOE_HIP(launch_combine(at<float>(ws, L.o), row_of, gate, shared_out, y, s.T, s.d, s.k, L.ksplit, (size_t)R * s.d,
                           st));
  MOE_MARK(MOE_NUM_STAGES);
#undef MOE_MARK
  return MOE_OK;
}

moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const void* w_r, const float* b_r,
                               const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
                               const void* ws_up, const void* ws_down, const moe_wscales* scales,
                               const moe_wscales* shared_scales, float* y, int32_t* idx, float* gate, int32_t* counts,
                               int32_t* kept, float* f, float* P, float* aux, int32_t* offsets, int32_t* row_token,
                               int32_t* row_of, void* stream, void* const* stage_events) {
  moe_status v = forward_args(shape, x, w_r, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, scales, shared_scales, y,
                              idx, gate, counts, kept, f, P, aux);
  if (v != MOE_OK) return v;
  if (layout(*shape).total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  v = static_scratch(&ws);
  if (v != MOE_OK) return v;
  // Every workspace byte the layer reads is written earlier in the same call, so the scratch
  // needs no clearing between calls.
  return moe_forward(shape, x, w_r, b_r, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, scales, shared_scales, y, idx,
                     gate, counts, kept, f, P, aux, offsets, row_token, row_of, ws, (size_t)MOE_STATIC_SCRATCH_BYTES,
                     stream, stage_events);
}

moe_status moe_mxfp8_quantize(int32_t rows, int32_t K, const void* x, uint8_t* codes, uint8_t* scales,
                              void* stream) {
  if (rows < 0 || K < 32 || K % 32 != 0) return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_ERR_NULL;
  MOE_HIP(launch_mxfp8_quantize(x, rows, K, codes, scales, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_backward_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->wfmt != MOE_W_NATIVE) return MOE_ERR_UNSUPPORTED;
  *bytes = bwd_layout(*shape).total;
  return MOE_OK;
}

moe_status moe_backward(const moe_shape* shape, const void* x, const void* w_r, const float* b_r, const void* w_gate,
                        const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                        const void* ws_down, const int32_t* idx, const float* gate, const int32_t* counts,
                        const int32_t* offsets, const int32_t* row_token, const int32_t* row_of, const float* dy,
                        float d_aux, float* dx, float* dw_r, float* db_r, float* dw_gate, float* dw_up,
                        float* dw_down, float* dws_gate, float* dws_up, float* dws_down, float* dgate, void* ws,
                        size_t ws_bytes, void* stream, void* const* stage_events) {
  moe_status v = check_shape(shape);
  if (v != MOE_OK) return v;
  const moe_shape& s = *shape;
  if (s.wfmt != MOE_W_NATIVE) return MOE_ERR_UNSUPPORTED;
  if (!w_r || !w_gate || !w_up || !w_down || !counts || !offsets || !dw_r || !dw_gate || !dw_up || !dw_down || !ws)
    return MOE_ERR_NULL;
  if (s.T > 0 && (!x || !idx || !gate || !row_token || !row_of || !dy || !dx)) return MOE_ERR_NULL;
  if (s.d_e_shared > 0 && (!ws_gate || !ws_up || !ws_down || !dws_gate || !dws_up || !dws_down)) return MOE_ERR_NULL;
  if (!isfinite(d_aux)) return MOE_ERR_SHAPE;
  const BwdLayout L = bwd_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  int next_stage = 0;
  auto mark = [&](int upto) -> bool {
    if (!stage_events) return true;
    for (; next_stage <= upto; ++next_stage)
      if (stage_events[next_stage] && hipEventRecord((hipEvent_t)stage_events[next_stage], st) != hipSuccess)
        return false;
    return true;
  };
#define MOE_MARK(i) \
  if (!mark(i)) return MOE_ERR_HIP

  const int T = s.T, d = s.d, de = s.d_e, des = s.d_e_shared, E = s.E;
  const long long R = (long long)T * s.k;
  const size_t es = elem_size(s.dtype);
  const GemmKind kind = L.kind;
  const int bm1 = gemm_block_m(kind, s.dtype, true, 0), bm2 = gemm_block_m(kind, s.dtype, false, 0);
  const int tiles1 = max_m_tiles(R, E, s.capacity, bm1), tiles2 = max_m_tiles(R, E, s.capacity, bm2);
  int32_t* poff = at<int32_t>(ws, L.poff);
  int32_t* koff_dense = at<int32_t>(ws, L.koff_dense);
  float* g_row = at<float>(ws, L.g_row);
  int32_t* ts1 = at<int32_t>(ws, L.ts1);   // tile starts of the gate/up-height tiles
  int32_t* ts2 = at<int32_t>(ws, L.ts2);   // ... and of the down-height tiles
  const void* dyb = s.dtype == MOE_BF16 ? at<void>(ws, L.dyb) : (const void*)dy;
  void* wdT = at<void>(ws, L.wdT);
  void* wguT = at<void>(ws, L.wguT);
  float* a = at<float>(ws, L.a);
  float* b = at<float>(ws, L.b);
  void* hT = at<void>(ws, L.hT);
  void* dab = at<void>(ws, L.dab);
  char* dabT = at<char>(ws, L.dabT);
  float* part = at<float>(ws, L.part);
  float* dr = at<float>(ws, L.dr);
  float* dX = at<float>(ws, L.dX);

  MOE_MARK(MOE_BSTAGE_PREP);
  MOE_HIP(launch_bwd_layout(offsets, E, row_of, gate, (int)R, poff, g_row, L.ldts, koff_dense, st));
  MOE_HIP(launch_transpose(s.dtype, w_down, E, d, de, wdT, d, 0, (size_t)de * d, st));
  MOE_HIP(launch_transpose(s.dtype, w_gate, E, de, d, wguT, 2 * de, 0, (size_t)d * 2 * de, st));
  MOE_HIP(launch_transpose(s.dtype, w_up, E, de, d, wguT, 2 * de, de, (size_t)d * 2 * de, st));
  if (s.dtype == MOE_BF16) MOE_HIP(launch_to_bf16(dy, (size_t)T * d, at<void>(ws, L.dyb), st));
  MOE_MARK(MOE_BSTAGE_RECOMPUTE);
  if (T > 0) {
    MOE_HIP(launch_tile_sched(offsets, E, bm1, ts1, bm2, ts2, st));
    MOE_HIP(launch_gemm_save_ab(kind, s.dtype, x, row_token, w_gate, w_up, offsets, ts1, E, 0, tiles1, de, d, a, b,
                                hT, poff, L.ldt, st));
    MOE_HIP(launch_zero_gaps(s.dtype, hT, de, L.ldt, offsets, poff, E, 0, 0, st));
  }
  MOE_MARK(MOE_BSTAGE_DOWN_BWD);
  if (T > 0) {
    MOE_HIP(launch_gemm_dgrad(kind, s.dtype, dyb, row_token, wdT, offsets, ts1, E, 0, tiles1, de, d, a, b, g_row, dab,
                              dabT, poff, L.ldt, part, st));
    MOE_HIP(launch_zero_gaps(s.dtype, dabT, 2 * de, L.ldt, offsets, poff, E, 0, 0, st));
  }
  MOE_MARK(MOE_BSTAGE_ROUTER_BWD);
  MOE_HIP(launch_router_bwd(s.dtype, x, w_r, b_r, T, d, E, s.k, s.renormalize, s.scoring, idx, gate, row_of, counts,
                            part, L.npart, d_aux, dr, dgate, at<float>(ws, L.logits), st));
  MOE_MARK(MOE_BSTAGE_DX_EXPERT);
  if (T > 0)
    MOE_HIP(launch_gemm_down(kind, s.dtype, 0, dab, wguT, nullptr, offsets, ts2, E, 0, tiles2, d, 2 * de, dX, 1, 0,
                             st, at<int32_t>(ws, L.tctr)));
  MOE_MARK(MOE_BSTAGE_WGRAD_DOWN);
  MOE_HIP(launch_gather_t(0, s.dtype, dy, d, row_token, g_row, offsets, poff, E, 0, L.ldt, at<void>(ws, L.doT), L.ldt,
                          st));
  MOE_HIP(launch_gemm_kgrouped(s.dtype, at<void>(ws, L.doT), hT, poff, E, d, de, L.ldt, dw_down, st));
  MOE_MARK(MOE_BSTAGE_WGRAD_GATE_UP);
  MOE_HIP(launch_gather_t(s.dtype, s.dtype, x, d, row_token, nullptr, offsets, poff, E, 0, L.ldt, at<void>(ws, L.xT),
                          L.ldt, st));
  MOE_HIP(launch_gemm_kgrouped(s.dtype, dabT, at<void>(ws, L.xT), poff, E, de, d, L.ldt, dw_gate, st));
  MOE_HIP(launch_gemm_kgrouped(s.dtype, dabT + (size_t)de * L.ldt * es, at<void>(ws, L.xT), poff, E, de, d, L.ldt,
                               dw_up, st));
  MOE_MARK(MOE_BSTAGE_SHARED);
  const float* sdX = nullptr;
  if (des > 0) {
    const GemmKind sk = L.skind;
    const int sbm1 = gemm_block_m(sk, s.dtype, true, 0), sbm2 = gemm_block_m(sk, s.dtype, false, 0);
    void* swdT = at<void>(ws, L.swdT);
    void* swguT = at<void>(ws, L.swguT);
    float* sa = at<float>(ws, L.sa);
    float* sb = at<float>(ws, L.sb);
    void* shT = at<void>(ws, L.shT);
    void* sdab = at<void>(ws, L.sdab);
    char* sdabT = at<char>(ws, L.sdabT);
    MOE_HIP(launch_transpose(s.dtype, ws_down, 1, d, des, swdT, d, 0, 0, st));
    MOE_HIP(launch_transpose(s.dtype, ws_gate, 1, des, d, swguT, 2 * des, 0, 0, st));
    MOE_HIP(launch_transpose(s.dtype, ws_up, 1, des, d, swguT, 2 * des, des, 0, st));
    if (T > 0) {
      MOE_HIP(launch_gemm_save_ab(sk, s.dtype, x, nullptr, ws_gate, ws_up, nullptr, nullptr, 1, T, (T + sbm1 - 1) / sbm1,
                                  des, d, sa, sb, shT, nullptr, L.ldts, st));
      MOE_HIP(launch_gemm_dgrad(sk, s.dtype, dyb, nullptr, swdT, nullptr, nullptr, 1, T, (T + sbm1 - 1) / sbm1, des, d,
                                sa, sb, nullptr, sdab, sdabT, nullptr, L.ldts, nullptr, st));
      MOE_HIP(launch_gemm_down(sk, s.dtype, 0, sdab, swguT, nullptr, nullptr, nullptr, 1, T, (T + sbm2 - 1) / sbm2, d,
                               2 * des, at<float>(ws, L.sdX), 1, 0, st));
      sdX = at<float>(ws, L.sdX);
    }
    MOE_HIP(launch_zero_gaps(s.dtype, shT, des, L.ldts, nullptr, nullptr, 1, T, L.ldts, st));
    MOE_HIP(launch_zero_gaps(s.dtype, sdabT, 2 * des, L.ldts, nullptr, nullptr, 1, T, L.ldts, st));
    MOE_HIP(launch_gather_t(0, s.dtype, dy, d, nullptr, nullptr, nullptr, nullptr, 1, T, L.ldts, at<void>(ws, L.sdyT),
                            L.ldts, st));
    MOE_HIP(launch_gather_t(s.dtype, s.dtype, x, d, nullptr, nullptr, nullptr, nullptr, 1, T, L.ldts,
                            at<void>(ws, L.sxT), L.ldts, st));
    MOE_HIP(launch_gemm_kgrouped(s.dtype, at<void>(ws, L.sdyT), shT, koff_dense, 1, d, des, L.ldts, dws_down, st));
    MOE_HIP(launch_gemm_kgrouped(s.dtype, sdabT, at<void>(ws, L.sxT), koff_dense, 1, des, d, L.ldts, dws_gate, st));
    MOE_HIP(launch_gemm_kgrouped(s.dtype, sdabT + (size_t)des * L.ldts * es, at<void>(ws, L.sxT), koff_dense, 1, des,
                                 d, L.ldts, dws_up, st));
  }
  MOE_MARK(MOE_BSTAGE_DX);
  MOE_HIP(launch_dx(s.dtype, dr, w_r, T, d, E, s.k, dX, row_of, sdX, dx, st));
  MOE_HIP(launch_dwr(s.dtype, dr, x, T, d, E, dw_r, db_r, s.scoring == MOE_SCORE_SIGMOID, at<float>(ws, L.dwr_part),
                     st));
  MOE_MARK(MOE_NUM_BSTAGES);
#undef MOE_MARK
  return MOE_OK;
}

}  // extern "C"
