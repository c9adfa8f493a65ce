// The C ABI (include/infini_attn.h): host-side validation, workspace layout
// and the launch plan. Nothing here touches device memory except through the
// kernels it enqueues; every check runs before the first launch.
//
// Plan. The segment recurrence has one sequential part, the (M, z) chain, and
// one parallel part, everything a segment does given the state before it
// ("Hugging Face Infini-Attention Reproduction Analysis", "Infini-Attention
// Mechanism": retrieval reads M_{s-1}; only the memory is carried). So a
// window of W segments runs as two launches on the caller's stream:
//   1. scan: walks the window's segments in order per (batch, KV head, slab of
//      M), writes the state before each segment into the workspace and the
//      state after the window;
//   2. attention: every (batch, query head, segment, query tile) of the window
//      in parallel, reading its segment's snapshot for the retrieval.
// W is as large as the workspace allows; with the full size the whole call is
// one window.
//
// The scan has two forms. The direct scan walks each segment's tokens in
// order (cost 6 N d^2 per segment on the sequential path, no extra memory).
// The affine form (affine.hip) computes each segment's d x d transition in
// parallel and leaves 2 d^3 per segment on the sequential path, at the price
// of two d x d matrices per segment in the workspace. It is used when
// seg_len >= 4 d, where its sequential part is at least 12x shorter.
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/infini_attn.h"
#include "kernels.hpp"

namespace {

using infini::AttnArgs;
using infini::AffineArgs;
using infini::ScanArgs;

constexpr int32_t kVersion = 100;  // 0.1.0
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int64_t units, S, d, e;
  bool affine;         // scan in affine form
  size_t state_bytes;  // one (M, z) buffer, aligned
  size_t per_seg;      // workspace bytes per segment of a window
  size_t fixed;        // bytes before the per-segment regions, plus alignment slack
};

bool use_affine(int64_t L, int64_t d, int64_t seg_len) {
  const int64_t eff = seg_len < L ? seg_len : L;
  return eff >= 4 * d;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

infini_status_t check_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d,
                            int64_t seg_len, int32_t rule, int32_t dtype, Plan* plan) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || d < 1 || seg_len < 1) return INFINI_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return INFINI_ERR_INVALID_ARG;
  if (rule != INFINI_RULE_LINEAR && rule != INFINI_RULE_DELTA) return INFINI_ERR_INVALID_ARG;
  if (dtype != INFINI_F32 && dtype != INFINI_BF16) return INFINI_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 128) return INFINI_ERR_UNSUPPORTED;
  // Every element index must fit in int64 and every grid in 2^31 workgroups.
  int64_t n = 0;
  if (!mul_ok(B, Hq, &n) || !mul_ok(n, L, &n) || !mul_ok(n, d, &n) || n > (INT64_MAX >> 3))
    return INFINI_ERR_INVALID_ARG;
  const int64_t units = B * Hkv;
  if (units * (d / 32) > INT32_MAX) return INFINI_ERR_INVALID_ARG;
  const int64_t S = (L + seg_len - 1) / seg_len;
  const int64_t eff = seg_len < L ? seg_len : L;
  const int64_t bm = 32 * infini::attn_waves(eff);
  const int64_t n_qt = (eff + bm - 1) / bm;
  // one segment per window at the least
  if (!mul_ok(B * Hq, n_qt, &n) || n > INT32_MAX) return INFINI_ERR_INVALID_ARG;
  if (plan) {
    plan->units = units;
    plan->S = S;
    plan->d = d;
    plan->e = dtype == INFINI_BF16 ? 2 : 4;
    plan->affine = use_affine(L, d, seg_len);
    plan->state_bytes = align_up((size_t)units * (size_t)(d * d + d) * 4);
    // snapshots: M^T in the element type, z in float
    size_t per = (size_t)(d * d * plan->e + d * 4);
    // affine form: column sums, B_s in float, A_s in the element type (delta)
    if (plan->affine)
      per += (size_t)(d * 4 + d * d * 4 + (rule == INFINI_RULE_DELTA ? d * d * plan->e : 0));
    plan->per_seg = (size_t)units * per;
    plan->fixed = 2 * plan->state_bytes + 6 * kAlign;
  }
  return INFINI_OK;
}

// Byte ranges [p, p + n) overlap.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace regions of a window of W segments: state A, state B (each (M, z)),
// then the window's snapshots and, for the affine form, its column sums and
// per-segment matrices.
struct Carved {
  float* stM[2];
  float* stz[2];
  void* snapM;
  float* snapZ;
  float* colsum;
  float* Bmat;
  void* Amat;
};

Carved carve(const Plan& p, int64_t W, int32_t rule, void* workspace) {
  Carved c{};
  char* ws = static_cast<char*>(workspace);
  const int64_t d = p.d;
  const size_t mbytes = (size_t)p.units * (size_t)(d * d) * 4;
  c.stM[0] = reinterpret_cast<float*>(ws);
  c.stM[1] = reinterpret_cast<float*>(ws + p.state_bytes);
  c.stz[0] = reinterpret_cast<float*>(ws + mbytes);
  c.stz[1] = reinterpret_cast<float*>(ws + p.state_bytes + mbytes);
  char* cur = ws + 2 * p.state_bytes;
  auto take = [&](size_t bytes) {
    char* r = cur;
    cur += align_up(bytes);
    return r;
  };
  const size_t uW = (size_t)p.units * (size_t)W;
  c.snapM = take(uW * (size_t)(d * d * p.e));
  c.snapZ = reinterpret_cast<float*>(take(uW * (size_t)d * 4));
  if (p.affine) {
    c.colsum = reinterpret_cast<float*>(take(uW * (size_t)d * 4));
    c.Bmat = reinterpret_cast<float*>(take(uW * (size_t)(d * d) * 4));
    if (rule == INFINI_RULE_DELTA) c.Amat = take(uW * (size_t)(d * d * p.e));
  }
  return c;
}

// The memory recurrence over segments [s_begin, s_begin + s_count) of k / v
// ([B*Hkv][L][d]), from (Min, zin) to (Mout, zout), writing the snapshots into
// the carved regions: the direct scan or the affine form, as the plan says.
hipError_t launch_recurrence(const Plan& p, const Carved& cw, int32_t rule, int32_t dtype,
                             const void* k, const void* v, const float* Min, const float* zin,
                             float* Mout, float* zout, int64_t L, int64_t seg_len,
                             int64_t s_begin, int64_t s_count, hipStream_t s) {
  if (p.affine) {
    AffineArgs fa;
    fa.k = k;
    fa.v = v;
    fa.M_in = Min;
    fa.z_in = zin;
    fa.M_out = Mout;
    fa.z_out = zout;
    fa.snapM = cw.snapM;
    fa.snapZ = cw.snapZ;
    fa.colsum = cw.colsum;
    fa.Amat = cw.Amat;
    fa.Bmat = cw.Bmat;
    fa.L = L;
    fa.seg_len = seg_len;
    fa.units = (int32_t)p.units;
    fa.s_begin = (int32_t)s_begin;
    fa.s_count = (int32_t)s_count;
    return infini::launch_affine(dtype, (int)p.d, rule, fa, s);
  }
  ScanArgs sa;
  sa.k = k;
  sa.v = v;
  sa.M_in = Min;
  sa.z_in = zin;
  sa.M_out = Mout;
  sa.z_out = zout;
  sa.snapM = cw.snapM;
  sa.snapZ = cw.snapZ;
  sa.L = L;
  sa.seg_len = seg_len;
  sa.units = (int32_t)p.units;
  sa.s_begin = (int32_t)s_begin;
  sa.s_count = (int32_t)s_count;
  return infini::launch_scan(dtype, (int)p.d, rule, sa, s);
}

}  // namespace

extern "C" {

infini_status_t infini_attn_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                           int64_t d, int64_t seg_len, int32_t rule,
                                           int32_t dtype, size_t* full_bytes,
                                           size_t* min_bytes) {
  Plan p;
  const infini_status_t st = check_sizes(B, Hq, Hkv, L, d, seg_len, rule, dtype, &p);
  if (st != INFINI_OK) return st;
  if (full_bytes) *full_bytes = p.fixed + p.per_seg * (size_t)p.S;
  if (min_bytes) *min_bytes = p.fixed + p.per_seg;
  return INFINI_OK;
}

}  // extern "C"

namespace {

infini_status_t forward_impl(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d,
                             int64_t seg_len, int32_t rule, int32_t dtype, const void* q,
                             const void* k, const void* v, const float* beta, const float* M0,
                             const float* z0, void* out, float* M_final, float* z_final,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events, int32_t n_events) {
  Plan p;
  infini_status_t st = check_sizes(B, Hq, Hkv, L, d, seg_len, rule, dtype, &p);
  if (st != INFINI_OK) return st;

  const void* ptrs[] = {q, k, v, beta, M0, z0, out, M_final, z_final, workspace};
  for (const void* ptr : ptrs) {
    if (ptr == nullptr) return INFINI_ERR_INVALID_ARG;
  }
  for (const void* ptr : ptrs) {
    if (!aligned16(ptr)) return INFINI_ERR_MISALIGNED;
  }

  const size_t nq = (size_t)(B * Hq * L * d) * (size_t)p.e;
  const size_t nkv = (size_t)(B * Hkv * L * d) * (size_t)p.e;
  const size_t nM = (size_t)(B * Hkv * d * d) * 4, nz = (size_t)(B * Hkv * d) * 4;
  const size_t nbeta = (size_t)Hq * 4;
  // out overlaps nothing; M_final / z_final may coincide exactly with M0 / z0;
  // the workspace overlaps nothing.
  struct Range { const void* p; size_t n; };
  const Range inputs[] = {{q, nq}, {k, nkv}, {v, nkv}, {beta, nbeta}, {M0, nM}, {z0, nz}};
  for (const Range& r : inputs) {
    if (overlap(out, nq, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (overlap(workspace, workspace_bytes, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (r.p != M0 && overlap(M_final, nM, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (r.p != z0 && overlap(z_final, nz, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
  }
  if (M0 != M_final && overlap(M_final, nM, M0, nM)) return INFINI_ERR_INVALID_ARG;
  if (z0 != z_final && overlap(z_final, nz, z0, nz)) return INFINI_ERR_INVALID_ARG;
  if (overlap(out, nq, M_final, nM) || overlap(out, nq, z_final, nz) ||
      overlap(M_final, nM, z_final, nz) || overlap(out, nq, workspace, workspace_bytes) ||
      overlap(workspace, workspace_bytes, M_final, nM) ||
      overlap(workspace, workspace_bytes, z_final, nz))
    return INFINI_ERR_INVALID_ARG;

  if (workspace_bytes < p.fixed + p.per_seg) return INFINI_ERR_WORKSPACE;
  int64_t W = (int64_t)((workspace_bytes - p.fixed) / p.per_seg);
  if (W > p.S) W = p.S;
  const int64_t eff = seg_len < L ? seg_len : L;
  const int64_t bm = 32 * infini::attn_waves(eff);
  const int64_t n_qt = (eff + bm - 1) / bm;
  const int64_t tiles_per_seg = B * Hq * n_qt;  // <= INT32_MAX, checked above
  if (W > INT32_MAX / tiles_per_seg) W = INT32_MAX / tiles_per_seg;

  const Carved cw = carve(p, W, rule, workspace);
  float* const* stM = cw.stM;
  float* const* stz = cw.stz;
  void* snapM = cw.snapM;
  float* snapZ = cw.snapZ;
  float* colsum = cw.colsum;
  float* Bmat = cw.Bmat;
  void* Amat = cw.Amat;

  if (n_events < 0 || (n_events > 0 && events == nullptr)) return INFINI_ERR_INVALID_ARG;
  for (int32_t e = 0; e < n_events; ++e)
    if (events[e] == nullptr) return INFINI_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Record event `slot` of window `wi` if the caller passed that many.
  auto mark = [&](int64_t wi, int slot) -> bool {
    const int64_t e = 3 * wi + slot;
    if (e >= n_events) return true;
    return hipEventRecord(static_cast<hipEvent_t>(events[e]), s) == hipSuccess;
  };
  const float* Min = M0;
  const float* zin = z0;
  if (z_final == z0 && !p.affine) {
    // In the direct scan several slab workgroups read z0 while one of them
    // writes z_final; read a copy instead. (The affine form reads and writes
    // each z entry in the same thread.)
    if (infini::launch_copy_f32(stz[1], z0, B * Hkv * d, s) != hipSuccess) return INFINI_ERR_HIP;
    zin = stz[1];
  }

  const int64_t n_windows = (p.S + W - 1) / W;
  for (int64_t wi = 0; wi < n_windows; ++wi) {
    const int64_t s_begin = wi * W;
    const int64_t s_count = (p.S - s_begin) < W ? (p.S - s_begin) : W;
    const bool last = wi == n_windows - 1;
    float* Mout = last ? M_final : stM[wi & 1];
    float* zout = last ? z_final : stz[wi & 1];

    if (!mark(wi, 0)) return INFINI_ERR_HIP;
    if (launch_recurrence(p, cw, rule, dtype, k, v, Min, zin, Mout, zout, L, seg_len, s_begin,
                          s_count, s) != hipSuccess)
      return INFINI_ERR_HIP;
    if (!mark(wi, 1)) return INFINI_ERR_HIP;

    AttnArgs aa;
    aa.q = q;
    aa.k = k;
    aa.v = v;
    aa.beta = beta;
    aa.snapM = snapM;
    aa.snapZ = snapZ;
    aa.out = out;
    aa.L = L;
    aa.seg_len = seg_len;
    aa.Hq = (int32_t)Hq;
    aa.Hkv = (int32_t)Hkv;
    aa.s_begin = (int32_t)s_begin;
    aa.s_count = (int32_t)s_count;
    aa.n_qt = (int32_t)n_qt;
    aa.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
    if (infini::launch_attn(dtype, (int)d, aa, p.units, s) != hipSuccess) return INFINI_ERR_HIP;
    if (!mark(wi, 2)) return INFINI_ERR_HIP;

    Min = Mout;
    zin = zout;
  }
  return INFINI_OK;
}

}  // namespace

extern "C" {

infini_status_t infini_attn_forward(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d,
                                    int64_t seg_len, int32_t rule, int32_t dtype,
                                    const void* q, const void* k, const void* v,
                                    const float* beta, const float* M0, const float* z0,
                                    void* out, float* M_final, float* z_final,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(B, Hq, Hkv, L, d, seg_len, rule, dtype, q, k, v, beta, M0, z0, out,
                      M_final, z_final, workspace, workspace_bytes, stream, nullptr, 0);
}

infini_status_t infini_attn_forward_timed(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                          int64_t d, int64_t seg_len, int32_t rule,
                                          int32_t dtype, const void* q, const void* k,
                                          const void* v, const float* beta, const float* M0,
                                          const float* z0, void* out, float* M_final,
                                          float* z_final, void* workspace,
                                          size_t workspace_bytes, void* stream,
                                          void* const* events, int32_t n_events) {
  return forward_impl(B, Hq, Hkv, L, d, seg_len, rule, dtype, q, k, v, beta, M0, z0, out,
                      M_final, z_final, workspace, workspace_bytes, stream, events, n_events);
}

// ---- streaming decode --------------------------------------------------------

}  // extern "C"

namespace {

struct DecodePlan {
  Plan fold;           // the recurrence over one segment of the cache
  int64_t G, n_chunks_max;
  size_t part_bytes;   // chunk partials, aligned
};

infini_status_t check_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t seg_len,
                             int32_t rule, int32_t dtype, DecodePlan* dp) {
  if (B < 1 || Hq < 1 || Hkv < 1 || d < 1 || seg_len < 1) return INFINI_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return INFINI_ERR_INVALID_ARG;
  if (Hq / Hkv > infini::kDecodeMaxGroup) return INFINI_ERR_UNSUPPORTED;
  if (seg_len > 64 * (int64_t)infini::kDecodeMaxChunks) return INFINI_ERR_UNSUPPORTED;
  Plan fold;
  const infini_status_t st = check_sizes(B, Hq, Hkv, seg_len, d, seg_len, rule, dtype, &fold);
  if (st != INFINI_OK) return st;
  if (fold.units * ((seg_len + 63) / 64) > INT32_MAX) return INFINI_ERR_INVALID_ARG;
  if (dp) {
    dp->fold = fold;
    dp->G = Hq / Hkv;
    dp->n_chunks_max = (seg_len + 63) / 64;
    dp->part_bytes = align_up((size_t)fold.units * (size_t)dp->n_chunks_max * (size_t)dp->G *
                              (size_t)(d + 2) * 4);
  }
  return INFINI_OK;
}

}  // namespace

extern "C" {

infini_status_t infini_attn_decode_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                                  int64_t seg_len, int32_t rule, int32_t dtype,
                                                  size_t* bytes) {
  DecodePlan dp;
  const infini_status_t st = check_decode(B, Hq, Hkv, d, seg_len, rule, dtype, &dp);
  if (st != INFINI_OK) return st;
  if (bytes) *bytes = dp.part_bytes + dp.fold.fixed + dp.fold.per_seg;
  return INFINI_OK;
}

infini_status_t infini_attn_decode_step(int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                        int64_t seg_len, int64_t pos, int32_t rule,
                                        int32_t dtype, const void* q, const void* k,
                                        const void* v, const float* beta, void* k_cache,
                                        void* v_cache, float* M, float* z, void* out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  DecodePlan dp;
  const infini_status_t st = check_decode(B, Hq, Hkv, d, seg_len, rule, dtype, &dp);
  if (st != INFINI_OK) return st;
  if (pos < 0 || pos >= seg_len) return INFINI_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, beta, k_cache, v_cache, M, z, out, workspace};
  for (const void* ptr : ptrs) {
    if (ptr == nullptr) return INFINI_ERR_INVALID_ARG;
  }
  for (const void* ptr : ptrs) {
    if (!aligned16(ptr)) return INFINI_ERR_MISALIGNED;
  }
  const Plan& p = dp.fold;
  const size_t e = (size_t)p.e;
  const size_t nq = (size_t)(B * Hq * d) * e, nkv = (size_t)(B * Hkv * d) * e;
  const size_t ncache = (size_t)(B * Hkv) * (size_t)seg_len * (size_t)d * e;
  const size_t nM = (size_t)(B * Hkv * d * d) * 4, nz = (size_t)(B * Hkv * d) * 4;
  struct Range { const void* p; size_t n; };
  const Range all[] = {{q, nq},           {k, nkv},           {v, nkv},
                       {beta, (size_t)Hq * 4}, {k_cache, ncache}, {v_cache, ncache},
                       {M, nM},           {z, nz},            {out, nq},
                       {workspace, workspace_bytes}};
  // the caches, the state, the output and the workspace are written: none of
  // them may overlap any other argument
  const int n_all = (int)(sizeof(all) / sizeof(all[0]));
  for (int x = 4; x < n_all; ++x)
    for (int y = 0; y < n_all; ++y)
      if (x != y && overlap(all[x].p, all[x].n, all[y].p, all[y].n)) return INFINI_ERR_INVALID_ARG;
  if (workspace_bytes < dp.part_bytes + p.fixed + p.per_seg) return INFINI_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  infini::DecodeArgs da;
  da.q = q;
  da.k = k;
  da.v = v;
  da.beta = beta;
  da.k_cache = k_cache;
  da.v_cache = v_cache;
  da.M = M;
  da.z = z;
  da.out = out;
  da.part = reinterpret_cast<float*>(ws);
  da.seg_len = seg_len;
  da.B = (int32_t)B;
  da.Hq = (int32_t)Hq;
  da.Hkv = (int32_t)Hkv;
  da.G = (int32_t)dp.G;
  da.pos = (int32_t)pos;
  da.n_chunks = (int32_t)((pos + 1 + 63) / 64);
  da.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  if (infini::launch_decode(dtype, (int)d, da, s) != hipSuccess) return INFINI_ERR_HIP;

  if (pos == seg_len - 1) {
    // the segment is complete: fold the cache into (M, z), in place
    const Carved cw = carve(p, 1, rule, ws + dp.part_bytes);
    const float* zin = z;
    if (!p.affine) {
      // the direct scan's slab workgroups read z while one of them writes it
      if (infini::launch_copy_f32(cw.stz[1], z, B * Hkv * d, s) != hipSuccess) return INFINI_ERR_HIP;
      zin = cw.stz[1];
    }
    if (launch_recurrence(p, cw, rule, dtype, k_cache, v_cache, M, zin, M, z, seg_len, seg_len, 0,
                          1, s) != hipSuccess)
      return INFINI_ERR_HIP;
  }
  return INFINI_OK;
}

const char* infini_attn_status_string(int32_t status) {
  switch (status) {
    case INFINI_OK: return "ok";
    case INFINI_ERR_INVALID_ARG: return "invalid argument";
    case INFINI_ERR_UNSUPPORTED: return "unsupported size (head dimension, group or segment length)";
    case INFINI_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case INFINI_ERR_WORKSPACE: return "workspace too small";
    case INFINI_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t infini_attn_version(void) { return kVersion; }

}  // extern "C"
