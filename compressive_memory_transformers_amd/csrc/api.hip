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
// of two d x d matrices per segment in the workspace (written once, read
// once). It is used when seg_len >= d: there its sequential part is at least
// 3x shorter and the matrices at most 1.5x the segment's K and V, and it was
// measured faster (2x at 128-token segments of d = 128); below, the
// matrices' traffic outgrows the tokens' and the direct scan is used.
#include <stdint.h>
#include <string.h>

#include <mutex>

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
  int64_t units, S, d, e;  // d: the key width (the value width too, unless dv says otherwise)
  int64_t dv;              // the value width
  bool affine;         // scan in affine form
  size_t state_bytes;  // one (M, z) buffer, aligned
  size_t per_seg;      // workspace bytes per segment of a window
  size_t fixed;        // bytes before the per-segment regions, plus alignment slack
};

bool use_affine(int64_t L, int64_t d, int64_t seg_len) {
  const int64_t eff = seg_len < L ? seg_len : L;
  return eff >= d;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Query rows per attention workgroup: the kernel with d_key != d_value
// always runs four waves.
int64_t attn_block_rows(int64_t dk, int64_t dv, int64_t eff) {
  return dk == dv ? 32 * infini::attn_waves(eff) : 128;
}

// dk: the key width, dv: the value width ("Infini-Attention" (AI Wiki), "How
// does the compressive memory work?": M is d_key x d_value).
infini_status_t check_sizes_kv(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t dk,
                               int64_t dv, int64_t seg_len, int32_t rule, int32_t dtype,
                               Plan* plan) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || dk < 1 || dv < 1 || seg_len < 1)
    return INFINI_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return INFINI_ERR_INVALID_ARG;
  if (rule != INFINI_RULE_LINEAR && rule != INFINI_RULE_DELTA) return INFINI_ERR_INVALID_ARG;
  if (dtype != INFINI_F32 && dtype != INFINI_BF16) return INFINI_ERR_INVALID_ARG;
  if (dk != 32 && dk != 64 && dk != 128) return INFINI_ERR_UNSUPPORTED;
  if (dv != 32 && dv != 64 && dv != 128) return INFINI_ERR_UNSUPPORTED;
  const int64_t d = dk > dv ? dk : dv;
  // Every element index must fit in int64 and every grid in 2^31 workgroups.
  int64_t n = 0;
  if (!mul_ok(B, Hq, &n) || !mul_ok(n, L, &n) || !mul_ok(n, d, &n) || n > (INT64_MAX >> 3))
    return INFINI_ERR_INVALID_ARG;
  const int64_t units = B * Hkv;
  if (units * (d / 32) > INT32_MAX) return INFINI_ERR_INVALID_ARG;
  const int64_t S = (L + seg_len - 1) / seg_len;
  const int64_t eff = seg_len < L ? seg_len : L;
  const int64_t bm = attn_block_rows(dk, dv, eff);
  const int64_t n_qt = (eff + bm - 1) / bm;
  // one segment per window at the least
  if (!mul_ok(B * Hq, n_qt, &n) || n > INT32_MAX) return INFINI_ERR_INVALID_ARG;
  if (plan) {
    plan->units = units;
    plan->S = S;
    plan->d = dk;
    plan->dv = dv;
    plan->e = dtype == INFINI_BF16 ? 2 : 4;
    // d_key != d_value: the direct scan only
    plan->affine = dk == dv && use_affine(L, dk, seg_len);
    plan->state_bytes = align_up((size_t)units * (size_t)(dk * dv + dk) * 4);
    // snapshots: M^T in the element type, z in float
    size_t per = (size_t)(dv * dk * plan->e + dk * 4);
    // affine form (dk == dv): column sums, B_s in float, A_s in the element type (delta)
    if (plan->affine)
      per += (size_t)(dk * 4 + dk * dk * 4 + (rule == INFINI_RULE_DELTA ? dk * dk * plan->e : 0));
    plan->per_seg = (size_t)units * per;
    plan->fixed = 2 * plan->state_bytes + 6 * kAlign;
  }
  return INFINI_OK;
}

infini_status_t check_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d,
                            int64_t seg_len, int32_t rule, int32_t dtype, Plan* plan) {
  return check_sizes_kv(B, Hq, Hkv, L, d, d, seg_len, rule, dtype, plan);
}

// Byte ranges [p, p + n) overlap.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace layout: state A, state B (each (M, z)), then one or two regions
// of per-segment data, each for a window of up to W segments: the window's
// snapshots and, for the affine form, its column sums and per-segment
// matrices.
struct Region {
  void* snapM;
  float* snapZ;
  float* colsum;
  float* Bmat;
  void* Amat;
};
struct Carved {
  float* stM[2];
  float* stz[2];
  Region r[2];
  Region head;  // one snapshot slot (overlapped plan): the state before segment 0
};

// Bytes of alignment slack that one region's sub-buffers can add.
constexpr size_t kRegionSlack = 5 * kAlign;

// Bytes of the head slot: one snapshot per unit, each part aligned.
size_t head_bytes(const Plan& p) {
  return align_up((size_t)p.units * (size_t)(p.dv * p.d * p.e)) +
         align_up((size_t)p.units * (size_t)p.d * 4);
}

// Workspace bytes for every segment at once: with more than one segment, the
// overlapped plan's two regions (S segments between them) and the head slot.
size_t workspace_full(const Plan& p) {
  if (p.S < 2) return p.fixed + p.per_seg;
  return p.fixed + kRegionSlack + head_bytes(p) + p.per_seg * (size_t)p.S;
}

// W0 segments in region 0, W1 (0: none) in region 1, and the head slot if
// `head`.
Carved carve(const Plan& p, int64_t W0, int64_t W1, int32_t rule, void* workspace,
             bool head = false) {
  Carved c{};
  char* ws = static_cast<char*>(workspace);
  const int64_t d = p.d, dv = p.dv;
  const size_t mbytes = (size_t)p.units * (size_t)(d * dv) * 4;
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
  const int64_t Ws[2] = {W0, W1};
  for (int ri = 0; ri < 2; ++ri) {
    if (Ws[ri] <= 0) continue;
    Region& g = c.r[ri];
    const size_t uW = (size_t)p.units * (size_t)Ws[ri];
    g.snapM = take(uW * (size_t)(dv * d * p.e));
    g.snapZ = reinterpret_cast<float*>(take(uW * (size_t)d * 4));
    if (p.affine) {
      g.colsum = reinterpret_cast<float*>(take(uW * (size_t)d * 4));
      g.Bmat = reinterpret_cast<float*>(take(uW * (size_t)(d * d) * 4));
      if (rule == INFINI_RULE_DELTA) g.Amat = take(uW * (size_t)(d * d * p.e));
    }
  }
  if (head) {
    c.head.snapM = take((size_t)p.units * (size_t)(dv * d * p.e));
    c.head.snapZ = reinterpret_cast<float*>(take((size_t)p.units * (size_t)d * 4));
  }
  return c;
}

// The auxiliary stream of the overlapped plan and its events, one set per
// device, created on first use and kept until the process ends (default
// priority, non-blocking). Calls enqueue under g_aux_mu, so concurrent calls
// never interleave their records and waits on these events.
struct Aux {
  bool tried = false, ok = false;
  hipStream_t s2 = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t rec[2] = {nullptr, nullptr};
  hipEvent_t att[2] = {nullptr, nullptr};
};
constexpr int kMaxDevices = 64;
std::mutex g_aux_mu;
Aux g_aux[kMaxDevices];

// The current device's set (null if it cannot be created); g_aux_mu held.
Aux* aux_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  Aux& a = g_aux[dev];
  if (!a.tried) {
    a.tried = true;
    bool ok = hipStreamCreateWithFlags(&a.s2, hipStreamNonBlocking) == hipSuccess;
    hipEvent_t* evs[] = {&a.start, &a.rec[0], &a.rec[1], &a.att[0], &a.att[1]};
    for (hipEvent_t* e : evs)
      ok = ok && hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess;
    a.ok = ok;
  }
  return a.ok ? &a : nullptr;
}

// The memory recurrence over segments [s_begin, s_begin + s_count) of k / v
// ([B*Hkv][L][d]), from (Min, zin) to (Mout, zout), writing the snapshots into
// the carved regions: the direct scan or the affine form, as the plan says.
hipError_t launch_recurrence(const Plan& p, const Region& cw, int32_t rule, int32_t dtype,
                             const void* k, const void* v, const float* Min, const float* zin,
                             float* Mout, float* zout, int64_t L, int64_t seg_len,
                             int64_t s_begin, int64_t s_count, hipStream_t s) {
  if (p.affine) {
    AffineArgs fa{};
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
    fa.reverse = 0;
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
  if (p.dv != p.d) return infini::launch_scan_kv(dtype, (int)p.d, (int)p.dv, rule, sa, s);
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
  if (full_bytes) *full_bytes = workspace_full(p);
  if (min_bytes) *min_bytes = p.fixed + p.per_seg;
  return INFINI_OK;
}

}  // extern "C"

namespace {

// d: the key width; dv: the value width (d for the square entry points).
infini_status_t forward_impl(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d,
                             int64_t seg_len, int32_t rule, int32_t dtype, const void* q,
                             const void* k, const void* v, const float* beta, const float* M0,
                             const float* z0, void* out, float* M_final, float* z_final,
                             float* lse, void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events, int32_t n_events, int64_t dv_in = 0,
                             bool allow_overlap = true) {
  const int64_t dv = dv_in > 0 ? dv_in : d;
  Plan p;
  infini_status_t st = check_sizes_kv(B, Hq, Hkv, L, d, dv, seg_len, rule, dtype, &p);
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
  const size_t nvv = (size_t)(B * Hkv * L * dv) * (size_t)p.e;
  const size_t nout = (size_t)(B * Hq * L * dv) * (size_t)p.e;
  const size_t nM = (size_t)(B * Hkv * d * dv) * 4, nz = (size_t)(B * Hkv * d) * 4;
  const size_t nbeta = (size_t)Hq * 4;
  // out overlaps nothing; M_final / z_final may coincide exactly with M0 / z0;
  // the workspace overlaps nothing.
  struct Range { const void* p; size_t n; };
  const Range inputs[] = {{q, nq}, {k, nkv}, {v, nvv}, {beta, nbeta}, {M0, nM}, {z0, nz}};
  for (const Range& r : inputs) {
    if (overlap(out, nout, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (overlap(workspace, workspace_bytes, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (r.p != M0 && overlap(M_final, nM, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (r.p != z0 && overlap(z_final, nz, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
  }
  if (M0 != M_final && overlap(M_final, nM, M0, nM)) return INFINI_ERR_INVALID_ARG;
  if (z0 != z_final && overlap(z_final, nz, z0, nz)) return INFINI_ERR_INVALID_ARG;
  if (overlap(out, nout, M_final, nM) || overlap(out, nout, z_final, nz) ||
      overlap(M_final, nM, z_final, nz) || overlap(out, nout, workspace, workspace_bytes) ||
      overlap(workspace, workspace_bytes, M_final, nM) ||
      overlap(workspace, workspace_bytes, z_final, nz))
    return INFINI_ERR_INVALID_ARG;
  if (lse != nullptr) {  // written: overlaps no other argument
    if (!aligned16(lse)) return INFINI_ERR_MISALIGNED;
    const size_t nl = (size_t)(B * Hq * L) * 4;
    for (const Range& r : inputs)
      if (overlap(lse, nl, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (overlap(lse, nl, out, nout) || overlap(lse, nl, M_final, nM) ||
        overlap(lse, nl, z_final, nz) || overlap(lse, nl, workspace, workspace_bytes))
      return INFINI_ERR_INVALID_ARG;
  }

  if (workspace_bytes < p.fixed + p.per_seg) return INFINI_ERR_WORKSPACE;
  if (n_events < 0 || (n_events > 0 && events == nullptr)) return INFINI_ERR_INVALID_ARG;
  for (int32_t e = 0; e < n_events; ++e)
    if (events[e] == nullptr) return INFINI_ERR_INVALID_ARG;
  const int64_t eff = seg_len < L ? seg_len : L;
  const int64_t bm = attn_block_rows(d, dv, eff);
  const int64_t n_qt = (eff + bm - 1) / bm;
  const int64_t tiles_per_seg = B * Hq * n_qt;  // <= INT32_MAX, checked above
  const int64_t max_launch = INT32_MAX / tiles_per_seg;  // segments per attention launch

  // Short segments (bf16, d in {64, 128}, Hq == Hkv, segments no longer than
  // d): the whole call in one pass, one workgroup per (batch, head) with the
  // state resident (fused.hip); the workspace is not used.
  if (dv == d && infini::fused_supported(dtype, (int)d, eff, Hq, Hkv)) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int slot = 0; slot < 2 && slot < n_events; ++slot)
      if (hipEventRecord(static_cast<hipEvent_t>(events[slot]), s) != hipSuccess)
        return INFINI_ERR_HIP;
    infini::FusedArgs fa;
    fa.q = q;
    fa.k = k;
    fa.v = v;
    fa.beta = beta;
    fa.M_in = M0;
    fa.z_in = z0;
    fa.M_out = M_final;
    fa.z_out = z_final;
    fa.out = out;
    fa.lse = lse;
    fa.L = L;
    fa.seg_len = (int32_t)eff;
    fa.H = (int32_t)Hq;
    fa.units = (int32_t)p.units;
    fa.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
    if (infini::launch_fused((int)d, rule, fa, s) != hipSuccess) return INFINI_ERR_HIP;
    if (n_events > 2 && hipEventRecord(static_cast<hipEvent_t>(events[2]), s) != hipSuccess)
      return INFINI_ERR_HIP;
    return INFINI_OK;
  }

  // Window plan. Serial: one region of W segments, each window's scan then
  // its attention on the caller's stream. Overlapped (the call has several
  // segments and two regions plus the head slot fit): segment 0's attention
  // starts at once from a snapshot of (M0, z0) in the head slot, while the
  // windows' scans run on an auxiliary stream into the two regions in turn,
  // and each window's attention (on the caller's stream) waits only for its
  // own window's scan. The scan's time on the critical path is then the part
  // segment 0's attention does not cover. It runs when the workspace has the
  // full size (workspace_full) and the scan is worth hiding (below): the
  // first window is S / 4 segments and the
  // second all the rest (more windows, alternating between the two regions,
  // only if a launch would exceed 2^31 workgroups). A smaller workspace runs
  // the serial plan, in one window if every segment's data fits.
  int64_t W = (int64_t)((workspace_bytes - p.fixed) / p.per_seg);
  if (W > p.S) W = p.S;
  if (W > max_launch) W = max_launch;
  int64_t C[2] = {W, 0};
  bool overlapped = false;
  std::unique_lock<std::mutex> lock(g_aux_mu, std::defer_lock);
  Aux* aux = nullptr;
  // The overlap pays where the scan is the direct form on a large call: a
  // latency-bound walk over the segments on few workgroups, which leaves the
  // attention room to run beside it (measured: d_key 64 / d_value 128 at the
  // Llama layer's sizes, 3.01 -> 2.68 ms per call). The affine form's scan is
  // mostly parallel work that competes with the attention for the whole chip
  // (measured 1-2% slower overlapped at the Llama layer and at 128-token
  // segments), and on small calls the extra launches and event waits cost
  // more than they hide; those run the serial plan. The exception is the
  // linear rule over many segments, whose state prefix is a walk over the
  // segments on few workgroups (measured at 512 segments of 2048 tokens,
  // d = 128: 13.63 -> 13.36 ms per call).
  const bool long_linear = p.affine && rule == INFINI_RULE_LINEAR && p.S >= 64;
  const bool worth_overlap =
      (!p.affine || long_linear) && (double)B * Hq * L * d >= (double)(1 << 26);
  if (allow_overlap && p.S >= 2 && worth_overlap && workspace_bytes >= workspace_full(p)) {
    int64_t c0 = p.S / 4 > 0 ? p.S / 4 : 1;
    int64_t c1 = p.S - c0;
    if (c0 > max_launch) c0 = max_launch;
    if (c1 > max_launch) c1 = max_launch;
    if (c0 >= 1 && c1 >= 1) {
      lock.lock();
      aux = aux_for_current_device();
      if (aux != nullptr) {
        overlapped = true;
        C[0] = c0;
        C[1] = c1;
      } else {
        lock.unlock();
      }
    }
  }

  const Carved cw = carve(p, C[0], C[1], rule, workspace, overlapped);
  float* const* stM = cw.stM;
  float* const* stz = cw.stz;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t sr = overlapped ? aux->s2 : s;  // the stream the scans run on
  // Caller event `slot`: 0 at the start, 1 before the first attention
  // kernel, 2 after the last one.
  auto mark = [&](int slot) -> bool {
    if (slot >= n_events) return true;
    return hipEventRecord(static_cast<hipEvent_t>(events[slot]), s) == hipSuccess;
  };
  // Segments [sb, sb + sc) of the attention, reading the snapshots of region
  // `rg` whose first entry is segment sb - first.
  auto attention = [&](const Region& rg, int64_t sb, int64_t sc, int64_t first,
                       int64_t count) -> bool {
    AttnArgs aa;
    aa.q = q;
    aa.k = k;
    aa.v = v;
    aa.beta = beta;
    aa.snapM = rg.snapM;
    aa.snapZ = rg.snapZ;
    aa.out = out;
    aa.lse = lse;
    aa.L = L;
    aa.seg_len = seg_len;
    aa.Hq = (int32_t)Hq;
    aa.Hkv = (int32_t)Hkv;
    aa.s_begin = (int32_t)sb;
    aa.s_count = (int32_t)sc;
    aa.snap_first = (int32_t)first;
    aa.snap_count = (int32_t)count;
    aa.n_qt = (int32_t)n_qt;
    aa.scale_log2 = 1.4426950408889634f / sqrtf((float)d);  // scores scale with the key width
    const hipError_t ea = dv == d ? infini::launch_attn(dtype, (int)d, aa, p.units, s)
                                  : infini::launch_attn_kv(dtype, (int)d, (int)dv, aa, p.units, s);
    return ea == hipSuccess;
  };
  if (!mark(0)) return INFINI_ERR_HIP;
  const float* Min = M0;
  const float* zin = z0;
  if (z_final == z0 && !p.affine) {
    // In the direct scan several slab workgroups read z0 while one of them
    // writes z_final; read a copy instead. (The affine form reads and writes
    // each z entry in the same thread.)
    if (infini::launch_copy_f32(stz[1], z0, B * Hkv * d, s) != hipSuccess) return INFINI_ERR_HIP;
    zin = stz[1];
  }
  if (overlapped) {
    // the head slot, read before the scans may overwrite M0 / z0 (in place)
    if (infini::launch_snapshot(dtype, (int)d, (int)dv, M0, zin, cw.head.snapM, cw.head.snapZ,
                                p.units, s) != hipSuccess)
      return INFINI_ERR_HIP;
    // the auxiliary stream starts after the caller's work so far
    if (hipEventRecord(aux->start, s) != hipSuccess ||
        hipStreamWaitEvent(sr, aux->start, 0) != hipSuccess)
      return INFINI_ERR_HIP;
    if (!mark(1)) return INFINI_ERR_HIP;
    if (!attention(cw.head, 0, 1, 0, 1)) return INFINI_ERR_HIP;
  }

  int64_t s_begin = 0;
  for (int64_t wi = 0; s_begin < p.S; ++wi) {
    const int ri = overlapped ? (int)(wi & 1) : 0;
    const int64_t s_count = (p.S - s_begin) < C[ri] ? (p.S - s_begin) : C[ri];
    const bool last = s_begin + s_count == p.S;
    float* Mout = last ? M_final : stM[wi & 1];
    float* zout = last ? z_final : stz[wi & 1];
    const Region& rg = cw.r[ri];

    // the region's previous window must have finished its attention
    if (overlapped && wi >= 2 && hipStreamWaitEvent(sr, aux->att[ri], 0) != hipSuccess)
      return INFINI_ERR_HIP;
    if (launch_recurrence(p, rg, rule, dtype, k, v, Min, zin, Mout, zout, L, seg_len, s_begin,
                          s_count, sr) != hipSuccess)
      return INFINI_ERR_HIP;
    if (overlapped && (hipEventRecord(aux->rec[ri], sr) != hipSuccess ||
                       hipStreamWaitEvent(s, aux->rec[ri], 0) != hipSuccess))
      return INFINI_ERR_HIP;
    if (!overlapped && wi == 0 && !mark(1)) return INFINI_ERR_HIP;
    // segment 0 already ran from the head slot in the overlapped plan
    const int64_t skip = overlapped && wi == 0 ? 1 : 0;
    if (s_count > skip && !attention(rg, s_begin + skip, s_count - skip, skip, s_count))
      return INFINI_ERR_HIP;
    if (overlapped && hipEventRecord(aux->att[ri], s) != hipSuccess) return INFINI_ERR_HIP;

    Min = Mout;
    zin = zout;
    s_begin += s_count;
  }
  if (!mark(2)) return INFINI_ERR_HIP;
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
                      M_final, z_final, nullptr, workspace, workspace_bytes, stream, nullptr, 0);
}

infini_status_t infini_attn_workspace_size_kv(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                              int64_t d_key, int64_t d_value, int64_t seg_len,
                                              int32_t rule, int32_t dtype, size_t* full_bytes,
                                              size_t* min_bytes) {
  Plan p;
  const infini_status_t st =
      check_sizes_kv(B, Hq, Hkv, L, d_key, d_value, seg_len, rule, dtype, &p);
  if (st != INFINI_OK) return st;
  if (full_bytes) *full_bytes = workspace_full(p);
  if (min_bytes) *min_bytes = p.fixed + p.per_seg;
  return INFINI_OK;
}

infini_status_t infini_attn_forward_kv(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                       int64_t d_key, int64_t d_value, int64_t seg_len,
                                       int32_t rule, int32_t dtype, const void* q, const void* k,
                                       const void* v, const float* beta, const float* M0,
                                       const float* z0, void* out, float* M_final,
                                       float* z_final, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (d_value < 1) return INFINI_ERR_INVALID_ARG;
  return forward_impl(B, Hq, Hkv, L, d_key, seg_len, rule, dtype, q, k, v, beta, M0, z0, out,
                      M_final, z_final, nullptr, workspace, workspace_bytes, stream, nullptr, 0,
                      d_value);
}

infini_status_t infini_attn_forward_kv_timed(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                             int64_t d_key, int64_t d_value, int64_t seg_len,
                                             int32_t rule, int32_t dtype, const void* q,
                                             const void* k, const void* v, const float* beta,
                                             const float* M0, const float* z0, void* out,
                                             float* M_final, float* z_final, void* workspace,
                                             size_t workspace_bytes, void* stream,
                                             void* const* events, int32_t n_events) {
  if (d_value < 1) return INFINI_ERR_INVALID_ARG;
  return forward_impl(B, Hq, Hkv, L, d_key, seg_len, rule, dtype, q, k, v, beta, M0, z0, out,
                      M_final, z_final, nullptr, workspace, workspace_bytes, stream, events,
                      n_events, d_value);
}

infini_status_t infini_attn_forward_train(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                          int64_t d, int64_t seg_len, int32_t rule,
                                          int32_t dtype, const void* q, const void* k,
                                          const void* v, const float* beta, const float* M0,
                                          const float* z0, void* out, float* M_final,
                                          float* z_final, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (lse == nullptr) return INFINI_ERR_INVALID_ARG;
  return forward_impl(B, Hq, Hkv, L, d, seg_len, rule, dtype, q, k, v, beta, M0, z0, out,
                      M_final, z_final, lse, workspace, workspace_bytes, stream, nullptr, 0);
}

infini_status_t infini_attn_forward_train_kv(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                             int64_t d_key, int64_t d_value, int64_t seg_len,
                                             int32_t rule, int32_t dtype, const void* q,
                                             const void* k, const void* v, const float* beta,
                                             const float* M0, const float* z0, void* out,
                                             float* M_final, float* z_final, float* lse,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (lse == nullptr || d_value < 1) return INFINI_ERR_INVALID_ARG;
  return forward_impl(B, Hq, Hkv, L, d_key, seg_len, rule, dtype, q, k, v, beta, M0, z0, out,
                      M_final, z_final, lse, workspace, workspace_bytes, stream, nullptr, 0,
                      d_value);
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
                      M_final, z_final, nullptr, workspace, workspace_bytes, stream, events,
                      n_events);
}

}  // extern "C"

// ---- the forward without a workspace ------------------------------------------
//
// For callers that cannot allocate: the workspace of infini_attn_forward is
// this array, one copy per GPU the library runs on, held until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory:
// the kernels get the address hipGetSymbolAddress returns for the current
// device (looked up on the first call on that device and kept), never the
// name. Nothing in it needs to start at zero: every workspace byte a forward
// reads was written earlier in the same call.
static_assert(INFINI_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[INFINI_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; null until looked up

// The current device's address of `scratch`, or null if the runtime cannot
// give it (then the next call asks again).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

infini_status_t infini_attn_forward_noalloc(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                            int64_t d, int64_t seg_len, int32_t rule,
                                            int32_t dtype, const void* q, const void* k,
                                            const void* v, const float* beta, const float* M0,
                                            const float* z0, void* out, float* M_final,
                                            float* z_final, void* stream) {
  Plan p;
  const infini_status_t st = check_sizes(B, Hq, Hkv, L, d, seg_len, rule, dtype, &p);
  if (st != INFINI_OK) return st;
  // the least workspace the call needs must fit the array
  if (p.fixed + p.per_seg > (size_t)INFINI_NOALLOC_SCRATCH_BYTES) return INFINI_ERR_WORKSPACE;
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return INFINI_ERR_HIP;
  // the serial plan only: no auxiliary stream, everything on `stream`
  return forward_impl(B, Hq, Hkv, L, d, seg_len, rule, dtype, q, k, v, beta, M0, z0, out,
                      M_final, z_final, nullptr, ws, INFINI_NOALLOC_SCRATCH_BYTES, stream,
                      nullptr, 0, 0, false);
}

// ---- streaming decode --------------------------------------------------------

}  // extern "C"

namespace {

struct DecodePlan {
  Plan fold;           // the recurrence over one segment of the cache
  int64_t G, n_chunks_max;
  size_t retr_off, rden_off;  // the retrieval's numerators and denominators
  size_t part_bytes;   // chunk partials and the retrieval, aligned
};

// d: the key width; dv: the value width (d when 0).
infini_status_t check_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t seg_len,
                             int32_t rule, int32_t dtype, DecodePlan* dp, int64_t dv = 0) {
  if (dv == 0) dv = d;
  if (B < 1 || Hq < 1 || Hkv < 1 || d < 1 || dv < 1 || seg_len < 1) return INFINI_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return INFINI_ERR_INVALID_ARG;
  if (Hq / Hkv > infini::kDecodeMaxGroup) return INFINI_ERR_UNSUPPORTED;
  if (seg_len > 64 * (int64_t)infini::kDecodeMaxChunks) return INFINI_ERR_UNSUPPORTED;
  Plan fold;
  const infini_status_t st =
      check_sizes_kv(B, Hq, Hkv, seg_len, d, dv, seg_len, rule, dtype, &fold);
  if (st != INFINI_OK) return st;
  if (fold.units * ((seg_len + 63) / 64) > INT32_MAX) return INFINI_ERR_INVALID_ARG;
  if (dp) {
    dp->fold = fold;
    dp->G = Hq / Hkv;
    dp->n_chunks_max = (seg_len + 63) / 64;
    dp->retr_off = align_up((size_t)fold.units * (size_t)dp->n_chunks_max * (size_t)dp->G *
                            (size_t)(dv + 2) * 4);
    dp->rden_off = dp->retr_off + align_up((size_t)fold.units * (size_t)dp->G * (size_t)dv * 4);
    dp->part_bytes = dp->rden_off + align_up((size_t)fold.units * (size_t)dp->G * 4);
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

}  // extern "C"

namespace {

// d: the key width; dv: the value width.
infini_status_t decode_impl(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t dv,
                            int64_t seg_len, int64_t pos, int32_t rule, int32_t dtype,
                            const void* q, const void* k, const void* v, const float* beta,
                            void* k_cache, void* v_cache, float* M, float* z, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  DecodePlan dp;
  const infini_status_t st = check_decode(B, Hq, Hkv, d, seg_len, rule, dtype, &dp, dv);
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
  const size_t nq = (size_t)(B * Hq * d) * e, nk = (size_t)(B * Hkv * d) * e;
  const size_t nv = (size_t)(B * Hkv * dv) * e, nout = (size_t)(B * Hq * dv) * e;
  const size_t nkc = (size_t)(B * Hkv) * (size_t)seg_len * (size_t)d * e;
  const size_t nvc = (size_t)(B * Hkv) * (size_t)seg_len * (size_t)dv * e;
  const size_t nM = (size_t)(B * Hkv * d * dv) * 4, nz = (size_t)(B * Hkv * d) * 4;
  struct Range { const void* p; size_t n; };
  const Range all[] = {{q, nq},           {k, nk},            {v, nv},
                       {beta, (size_t)Hq * 4}, {k_cache, nkc}, {v_cache, nvc},
                       {M, nM},           {z, nz},            {out, nout},
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
  da.retr = reinterpret_cast<float*>(ws + dp.retr_off);
  da.rden = reinterpret_cast<float*>(ws + dp.rden_off);
  da.seg_len = seg_len;
  da.B = (int32_t)B;
  da.Hq = (int32_t)Hq;
  da.Hkv = (int32_t)Hkv;
  da.G = (int32_t)dp.G;
  da.pos = (int32_t)pos;
  da.n_chunks = (int32_t)((pos + 1 + 63) / 64);
  da.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  if (infini::launch_decode_kv(dtype, (int)d, (int)dv, da, s) != hipSuccess) return INFINI_ERR_HIP;

  if (pos == seg_len - 1) {
    // the segment is complete: fold the cache into (M, z), in place
    const Carved cw = carve(p, 1, 0, rule, ws + dp.part_bytes);
    const float* zin = z;
    if (!p.affine) {
      // the direct scan's slab workgroups read z while one of them writes it
      if (infini::launch_copy_f32(cw.stz[1], z, B * Hkv * d, s) != hipSuccess) return INFINI_ERR_HIP;
      zin = cw.stz[1];
    }
    if (launch_recurrence(p, cw.r[0], rule, dtype, k_cache, v_cache, M, zin, M, z, seg_len, seg_len, 0,
                          1, s) != hipSuccess)
      return INFINI_ERR_HIP;
  }
  return INFINI_OK;
}

}  // namespace

extern "C" {

infini_status_t infini_attn_decode_step(int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                        int64_t seg_len, int64_t pos, int32_t rule,
                                        int32_t dtype, const void* q, const void* k,
                                        const void* v, const float* beta, void* k_cache,
                                        void* v_cache, float* M, float* z, void* out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(B, Hq, Hkv, d, d, seg_len, pos, rule, dtype, q, k, v, beta, k_cache,
                     v_cache, M, z, out, workspace, workspace_bytes, stream);
}

infini_status_t infini_attn_decode_workspace_size_kv(int64_t B, int64_t Hq, int64_t Hkv,
                                                     int64_t d_key, int64_t d_value,
                                                     int64_t seg_len, int32_t rule, int32_t dtype,
                                                     size_t* bytes) {
  if (d_value < 1) return INFINI_ERR_INVALID_ARG;
  DecodePlan dp;
  const infini_status_t st = check_decode(B, Hq, Hkv, d_key, seg_len, rule, dtype, &dp, d_value);
  if (st != INFINI_OK) return st;
  if (bytes) *bytes = dp.part_bytes + dp.fold.fixed + dp.fold.per_seg;
  return INFINI_OK;
}

infini_status_t infini_attn_decode_step_kv(int64_t B, int64_t Hq, int64_t Hkv, int64_t d_key,
                                           int64_t d_value, int64_t seg_len, int64_t pos,
                                           int32_t rule, int32_t dtype, const void* q,
                                           const void* k, const void* v, const float* beta,
                                           void* k_cache, void* v_cache, float* M, float* z,
                                           void* out, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (d_value < 1) return INFINI_ERR_INVALID_ARG;
  return decode_impl(B, Hq, Hkv, d_key, d_value, seg_len, pos, rule, dtype, q, k, v, beta,
                     k_cache, v_cache, M, z, out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- backward pass -------------------------------------------------------------
//
// Plan (kernels in bwd.hip, affine.hip): one window, the whole call.
//   1. the forward recurrence in affine form, for the states before each
//      segment (snapshots) and, with the delta rule, each segment's A_s;
//   2. retrieval: nm = sigma(Q) M_{s-1} (product), the row step (delta, dg,
//      dn, dden), nm = dn M_{s-1}^T (product), the retrieval part of dQ;
//      C_s = sum over the group's heads of sigma(Q)^T dn (products), and the
//      retrieval part of dL/dz_{s-1};
//   3. dM_s for every segment by the chain run backwards from dM_final,
//      dM_{s-1} = dM_s + A_s dM_s + C_s (A_s = 0 with the linear rule); dM0.
//      In float for every element type, with A_s formed in float: with a
//      small z_{s-1} the transition has large entries and would amplify bf16
//      rounding into dM0;
//   4. local attention: dK, dV (stored in float) and dQ;
//   5. update: Phi dM_s, the delta rule's Phi M_{s-1} and row step, then
//      dPhi = (U or V) dM_s^T (+ dP M_{s-1}^T) (products);
//   6. dz recurrence backwards from dz_final, the final dK, dV, and dbeta.

namespace {

struct BwdLayout {
  size_t total;
  size_t stM, stz, zeroM, snapM, snapZ, colsum, Bmat, Amat, dMsnap, e_ret, e_upd, dzs;
  size_t nm, dn, delta, dg, dden, dk_acc, dv_acc, du_buf, dphi, p_buf, u_el, dp_el, dc;
  size_t Amat_f, dMsnap_f, phi_f, phic_f, wsum_part, dbeta_part;
};

// fused: the bf16 kernels that form sigma(Q) M, sigma(K) dM_s and sigma(K)
// M_{s-1} in registers run (attn_bwd_mfma_supported), so the float row
// buffers of the product path (nm, du_buf, p_buf, u_el, dp_el) are not taken.
BwdLayout bwd_layout(const Plan& p, int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                     int64_t seg_len, int32_t rule, bool fused) {
  BwdLayout b{};
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t r = cur;
    cur += align_up(bytes);
    return r;
  };
  // d: the key width, dv: the value width; M-shaped buffers are d x dv
  const size_t d = (size_t)p.d, dv = (size_t)p.dv, e = (size_t)p.e, units = (size_t)p.units,
               S = (size_t)p.S;
  const size_t dmax = d > dv ? d : dv;
  const size_t qrows = (size_t)(B * Hq * L), krows = (size_t)(B * Hkv * L);
  const bool delta = rule == INFINI_RULE_DELTA;
  b.stM = take(units * d * dv * 4);
  b.stz = take(units * d * 4);
  b.zeroM = take(units * d * dv * 4);
  b.snapM = take(units * S * d * dv * e);
  b.snapZ = take(units * S * d * 4);
  b.colsum = take(units * S * d * 4);
  b.Bmat = take(units * S * d * dv * 4);
  b.Amat = delta ? take(units * S * d * d * e) : 0;
  b.dMsnap = take(units * S * d * dv * e);
  b.dMsnap_f = take(units * S * d * dv * 4);
  b.Amat_f = delta ? take(units * S * d * d * 4) : 0;
  b.e_ret = take(units * S * d * 4);
  b.e_upd = take(units * S * d * 4);
  b.dzs = take(units * S * d * 4);
  {  // chunks of 512 rows of a segment's query rows (all heads of the group)
    const size_t n = (size_t)(seg_len < L ? seg_len : L);
    const size_t chunks = ((size_t)(Hq / Hkv) * n + 511) / 512;
    b.wsum_part = take(units * S * chunks * d * 4);
  }
  b.dbeta_part =
      take((size_t)(Hq * B) * (size_t)((L + infini::kDbetaChunk - 1) / infini::kDbetaChunk) * 4);
  if (!fused) b.nm = take(qrows * dmax * 4);  // sigma(Q) M (dv), then dQ's retrieval part (d)
  b.dn = take(qrows * dv * e);
  b.delta = take(qrows * 4);
  b.dg = take(qrows * 4);
  b.dden = take(qrows * 4);
  b.dk_acc = take(krows * d * 4);
  b.dv_acc = take(krows * dv * 4);
  if (!fused) b.du_buf = take(krows * dv * 4);
  b.dphi = take(krows * d * 4);
  if (delta) {
    if (!fused) {
      b.p_buf = take(krows * dv * 4);
      b.u_el = take(krows * dv * e);
      b.dp_el = take(krows * dv * e);
    }
    b.dc = take(krows * 4);
    if (!infini::affine_a_f32_supported(p.e == 2 ? infini::kBF16 : infini::kF32, (int)d)) {
      b.phi_f = take(krows * d * 4);
      b.phic_f = take(krows * d * 4);
    }
  }
  b.total = cur + kAlign;  // slack for an unaligned base
  return b;
}

// A product over the (hi, lo) batches: hi = B * heads rows of a [.][L][d]
// tensor, lo = the segment. Defaults: no transposes, alpha 1, overwrite.
infini::GemmArgs gemm_args(const void* A, const void* B, float* C, int32_t M, int32_t N,
                           int32_t K, int64_t hi_count, int64_t S, int64_t L, int64_t seg_len) {
  infini::GemmArgs g{};
  g.A = A;
  g.B = B;
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.alpha = 1.f;
  g.batches = (int32_t)(hi_count * S);
  g.S = (int32_t)S;
  g.a_div = g.b_div = g.c_div = 1;
  g.L = L;
  g.seg_len = seg_len;
  return g;
}

infini_status_t backward_workspace_impl(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d,
                                       int64_t dv, int64_t seg_len, int32_t rule, int32_t dtype,
                                       size_t* bytes) {
  Plan p;
  const infini_status_t st = check_sizes_kv(B, Hq, Hkv, L, d, dv, seg_len, rule, dtype, &p);
  if (st != INFINI_OK) return st;
  if ((int64_t)p.units * p.S > INT32_MAX || B * Hq * p.S > INT32_MAX) return INFINI_ERR_INVALID_ARG;
  const bool fused = d == dv && infini::attn_bwd_mfma_supported(dtype, (int)d, (int)(Hq / Hkv));
  if (bytes) *bytes = bwd_layout(p, B, Hq, Hkv, L, seg_len, rule, fused).total;
  return INFINI_OK;
}

}  // namespace

extern "C" {

infini_status_t infini_attn_backward_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                                    int64_t d, int64_t seg_len, int32_t rule,
                                                    int32_t dtype, size_t* bytes) {
  return backward_workspace_impl(B, Hq, Hkv, L, d, d, seg_len, rule, dtype, bytes);
}

infini_status_t infini_attn_backward_workspace_size_kv(int64_t B, int64_t Hq, int64_t Hkv,
                                                       int64_t L, int64_t d_key, int64_t d_value,
                                                       int64_t seg_len, int32_t rule,
                                                       int32_t dtype, size_t* bytes) {
  if (d_value < 1) return INFINI_ERR_INVALID_ARG;
  return backward_workspace_impl(B, Hq, Hkv, L, d_key, d_value, seg_len, rule, dtype, bytes);
}

}  // extern "C"

namespace {

// d: the key width, dv: the value width ("Infini-Attention" (AI Wiki), "How
// does the compressive memory work?": M is d_key x d_value).
infini_status_t backward_impl(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t dv,
                              int64_t seg_len, int32_t rule, int32_t dtype, const void* q,
                              const void* k, const void* v, const float* beta, const float* M0,
                              const float* z0, const void* out, const float* lse,
                              const void* d_out, const float* dM_final, const float* dz_final,
                              void* dq, void* dk, void* dvv, float* dbeta, float* dM0,
                              float* dz0, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Plan p;
  infini_status_t st = check_sizes_kv(B, Hq, Hkv, L, d, dv, seg_len, rule, dtype, &p);
  if (st != INFINI_OK) return st;
  if ((int64_t)p.units * p.S > INT32_MAX || B * Hq * p.S > INT32_MAX) return INFINI_ERR_INVALID_ARG;
  const void* required[] = {q, k, v, beta, M0, z0, out, lse, d_out, dq, dk, dvv, dbeta, dM0, dz0,
                            workspace};
  for (const void* ptr : required)
    if (ptr == nullptr) return INFINI_ERR_INVALID_ARG;
  for (const void* ptr : required)
    if (!aligned16(ptr)) return INFINI_ERR_MISALIGNED;
  if ((dM_final && !aligned16(dM_final)) || (dz_final && !aligned16(dz_final)))
    return INFINI_ERR_MISALIGNED;
  const size_t e = (size_t)p.e;
  const size_t nq = (size_t)(B * Hq * L * d) * e, nk = (size_t)(B * Hkv * L * d) * e;
  const size_t nv = (size_t)(B * Hkv * L * dv) * e, no = (size_t)(B * Hq * L * dv) * e;
  const size_t nM = (size_t)(B * Hkv * d * dv) * 4, nz = (size_t)(B * Hkv * d) * 4;
  const size_t nrow = (size_t)(B * Hq * L) * 4, nbeta = (size_t)Hq * 4;
  const bool bwd_mfma = d == dv && infini::attn_bwd_mfma_supported(dtype, (int)d, (int)(Hq / Hkv));
  const BwdLayout lay = bwd_layout(p, B, Hq, Hkv, L, seg_len, rule, bwd_mfma);
  if (workspace_bytes < lay.total) return INFINI_ERR_WORKSPACE;
  struct Range { const void* p; size_t n; };
  const Range all[] = {{q, nq},         {k, nk},          {v, nv},       {beta, nbeta},
                       {M0, nM},        {z0, nz},         {out, no},     {lse, nrow},
                       {d_out, no},     {dM_final, nM},   {dz_final, nz}, {dq, nq},
                       {dk, nk},        {dvv, nv},        {dbeta, nbeta}, {dM0, nM},
                       {dz0, nz},       {workspace, workspace_bytes}};
  // the outputs and the workspace (from entry 11 on) overlap no other argument
  const int n_all = (int)(sizeof(all) / sizeof(all[0]));
  for (int x = 11; x < n_all; ++x)
    for (int y = 0; y < n_all; ++y)
      if (x != y && all[y].p != nullptr && overlap(all[x].p, all[x].n, all[y].p, all[y].n))
        return INFINI_ERR_INVALID_ARG;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(align_up((size_t)(uintptr_t)workspace) -
                                     (size_t)(uintptr_t)workspace + static_cast<char*>(workspace));
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  auto E = [&](size_t off) { return static_cast<void*>(ws + off); };
  const int64_t S = p.S, units = p.units, G = Hq / Hkv;
  const int32_t D = (int32_t)d, DV = (int32_t)dv;
  const int32_t N = (int32_t)(seg_len < L ? seg_len : L);  // rows of the longest segment

  // 1. states before each segment: the affine form (one width), or the
  // direct scan (two widths)
  AffineArgs fa{};
  fa.k = k;
  fa.v = v;
  fa.M_in = M0;
  fa.z_in = z0;
  fa.M_out = F(lay.stM);
  fa.z_out = F(lay.stz);
  fa.snapM = E(lay.snapM);
  fa.snapZ = F(lay.snapZ);
  fa.colsum = F(lay.colsum);
  fa.Amat = rule == INFINI_RULE_DELTA ? E(lay.Amat) : nullptr;
  fa.Bmat = F(lay.Bmat);
  fa.L = L;
  fa.seg_len = seg_len;
  fa.units = (int32_t)units;
  fa.s_begin = 0;
  fa.s_count = (int32_t)S;
  fa.reverse = 0;
  if (d == dv) {
    if (infini::launch_affine(dtype, D, rule, fa, s) != hipSuccess) return INFINI_ERR_HIP;
  } else {
    ScanArgs sa;
    sa.k = k;
    sa.v = v;
    sa.M_in = M0;
    sa.z_in = z0;
    sa.M_out = F(lay.stM);
    sa.z_out = F(lay.stz);
    sa.snapM = E(lay.snapM);
    sa.snapZ = F(lay.snapZ);
    sa.L = L;
    sa.seg_len = seg_len;
    sa.units = (int32_t)units;
    sa.s_begin = 0;
    sa.s_count = (int32_t)S;
    if (infini::launch_scan_kv(dtype, D, DV, rule, sa, s) != hipSuccess) return INFINI_ERR_HIP;
  }

  infini::BwdArgs ba{};
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.beta = beta;
  ba.out = out;
  ba.lse = lse;
  ba.dout = d_out;
  ba.snapM = E(lay.snapM);
  ba.snapZ = F(lay.snapZ);
  ba.nm = bwd_mfma ? nullptr : F(lay.nm);
  ba.dn = E(lay.dn);
  ba.delta = F(lay.delta);
  ba.dg = F(lay.dg);
  ba.dden = F(lay.dden);
  ba.dk_acc = F(lay.dk_acc);
  ba.dv_acc = F(lay.dv_acc);
  const bool rows = !bwd_mfma && rule == INFINI_RULE_DELTA;  // delta rule, product path
  ba.p_buf = rows ? F(lay.p_buf) : nullptr;
  ba.du_buf = bwd_mfma ? nullptr : F(lay.du_buf);
  ba.dphi = F(lay.dphi);
  ba.u_el = rows ? E(lay.u_el) : nullptr;
  ba.dp_el = rows ? E(lay.dp_el) : nullptr;
  ba.dc = rule == INFINI_RULE_DELTA ? F(lay.dc) : nullptr;
  ba.phi_f = rule == INFINI_RULE_DELTA && lay.phi_f ? F(lay.phi_f) : nullptr;
  ba.phic_f = rule == INFINI_RULE_DELTA && lay.phic_f ? F(lay.phic_f) : nullptr;
  ba.e_ret = F(lay.e_ret);
  ba.e_upd = F(lay.e_upd);
  ba.dzs = F(lay.dzs);
  ba.wsum_part = F(lay.wsum_part);
  ba.dbeta_part = F(lay.dbeta_part);
  ba.dz_final = dz_final;
  ba.dz0 = dz0;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dvv;
  ba.dbeta = dbeta;
  ba.L = L;
  ba.seg_len = seg_len;
  ba.B = (int32_t)B;
  ba.Hq = (int32_t)Hq;
  ba.Hkv = (int32_t)Hkv;
  ba.S = (int32_t)S;
  ba.rule = rule;
  ba.scale_log2 = 1.4426950408889634f / sqrtf((float)d);

  // row strides: key side (q, k) d, value side (v, out, dn, M's columns) dv
  const int64_t LD = L * d, ND = seg_len * d, LV = L * dv, NV = seg_len * dv, DDV = d * dv;
  // 2. retrieval. bf16 with d in {64, 128}: one fused kernel per 128 query
  // rows. Otherwise two products and a row kernel (query-side products:
  // hi = b * Hq + h, M_{s-1} of unit hi / G).
  if (bwd_mfma) {
    if (infini::launch_bwd_retrieval_mfma(D, ba, s) != hipSuccess) return INFINI_ERR_HIP;
  } else {
    {  // nm = sigma(Q) M, [rows][dv]
      infini::GemmArgs g = gemm_args(q, E(lay.snapM), ba.nm, N, DV, D, B * Hq, S, L, seg_len);
      g.lda = D;
      g.ldb = D;
      g.ldc = DV;
      g.a_hi = LD;
      g.a_lo = ND;
      g.c_hi = LV;
      g.c_lo = NV;
      g.b_div = (int32_t)G;
      g.b_hi = S * DDV;
      g.b_lo = DDV;
      g.tb = 1;  // op(B) = M, stored as M^T [dv][d]
      g.a_sigma = 1;
      g.clip = 1;
      if (infini::launch_gemm(dtype, g, s) != hipSuccess) return INFINI_ERR_HIP;
    }
    if (infini::launch_bwd_retrieval_rows(dtype, D, DV, ba, s) != hipSuccess)
      return INFINI_ERR_HIP;
    {  // nm = dQ's retrieval part, [rows][d]
      infini::GemmArgs g = gemm_args(ba.dn, E(lay.snapM), ba.nm, N, D, DV, B * Hq, S, L, seg_len);
      g.lda = DV;
      g.ldb = D;
      g.ldc = D;
      g.a_hi = LV;
      g.a_lo = NV;
      g.c_hi = LD;
      g.c_lo = ND;
      g.b_div = (int32_t)G;
      g.b_hi = S * DDV;
      g.b_lo = DDV;
      g.tb = 0;  // op(B) = M^T as stored
      g.clip = 1;
      // epilogue: nm = (dn M^T + dden z^T) sigma'(Q), the retrieval part of dQ
      g.epi = 1;
      g.epi_w = ba.dden;
      g.w_hi = L;
      g.w_lo = seg_len;
      g.epi_z = F(lay.snapZ);
      g.z_div = (int32_t)G;
      g.z_hi = S * d;
      g.z_lo = d;
      g.epi_x = q;
      if (infini::launch_gemm(dtype, g, s) != hipSuccess) return INFINI_ERR_HIP;
    }
  }
  // C_s = sum over the group's heads of sigma(Q)^T dn, into Bmat: bf16 with
  // d = 128 by the recurrence's product kernel (one pass over q and dn, which
  // also forms the retrieval part of dL/dz_{s-1}, sum of dden_t sigma(q_t),
  // from the rows it stages), otherwise one product per head, accumulating,
  // and a row reduction for the dz part
  if (dtype == INFINI_BF16 && d == 128 && dv == 128) {
    AffineArgs ca{};
    ca.k = q;
    ca.v = E(lay.dn);
    ca.snapZ = F(lay.snapZ);
    ca.Bmat = F(lay.Bmat);
    ca.colsum = F(lay.e_ret);
    ca.colsum_w = ba.dden;
    ca.L = L;
    ca.seg_len = seg_len;
    ca.units = (int32_t)units;
    ca.s_begin = 0;
    ca.s_count = (int32_t)S;
    ca.heads = (int32_t)G;
    if (infini::launch_affine_products(dtype, D, ca, s) != hipSuccess) return INFINI_ERR_HIP;
  } else {
    for (int64_t hg = 0; hg < G; ++hg) {  // C_s into Bmat, summed over the group's heads
      infini::GemmArgs g = gemm_args(static_cast<const char*>(q) + (size_t)(hg * LD) * e,
                                     static_cast<const char*>(E(lay.dn)) + (size_t)(hg * LV) * e,
                                     F(lay.Bmat), D, DV, (int32_t)seg_len, units, S, L, seg_len);
      g.lda = D;
      g.ldb = DV;
      g.ldc = DV;
      g.a_hi = G * LD;
      g.a_lo = ND;
      g.b_hi = G * LV;
      g.b_lo = NV;
      g.c_hi = S * DDV;
      g.c_lo = DDV;
      g.ta = 1;  // op(A) = sigma(Q)^T
      g.a_sigma = 1;
      g.clip = 2;
      g.accumulate = hg > 0;
      if (infini::launch_gemm(dtype, g, s) != hipSuccess) return INFINI_ERR_HIP;
    }
    if (infini::launch_bwd_row_weighted_sum(dtype, D, DV, ba, true, s) != hipSuccess)
      return INFINI_ERR_HIP;
  }

  // 3. dM_s for every segment, and dM0, in float. A_s = -Phi^T diag(1/c) Phi
  // from float sigma(K) and sigma(K) / c (bf16 with d = 128: from bf16 hi/lo
  // pairs of both, formed on the fly from K).
  if (rule == INFINI_RULE_DELTA && infini::affine_a_f32_supported(dtype, D)) {
    // bf16, d = 128: one pass over K, Phi and Phi / den split into bf16
    // pairs on three bf16 products per tile (affine.hip)
    AffineArgs aa = fa;
    aa.Amat_f = F(lay.Amat_f);
    if (infini::launch_affine_a_f32(aa, s) != hipSuccess) return INFINI_ERR_HIP;
  } else if (rule == INFINI_RULE_DELTA) {
    if (infini::launch_bwd_phi_rows(dtype, D, DV, ba, s) != hipSuccess) return INFINI_ERR_HIP;
    infini::GemmArgs g = gemm_args(ba.phi_f, ba.phic_f, F(lay.Amat_f), D, D, (int32_t)seg_len,
                                   units, S, L, seg_len);
    g.lda = g.ldb = g.ldc = D;
    g.a_hi = g.b_hi = LD;
    g.a_lo = g.b_lo = ND;
    g.c_hi = S * d * d;
    g.c_lo = d * d;
    g.ta = 1;  // op(A) = Phi^T
    g.alpha = -1.f;
    g.clip = 2;
    if (infini::launch_gemm(INFINI_F32, g, s) != hipSuccess) return INFINI_ERR_HIP;
  }
  const float* dM_in = dM_final;
  if (dM_in == nullptr) {
    if (infini::launch_fill_f32(F(lay.zeroM), 0.f, units * d * dv, s) != hipSuccess)
      return INFINI_ERR_HIP;
    dM_in = F(lay.zeroM);
  }
  AffineArgs ra = fa;
  ra.M_in = dM_in;
  ra.M_out = dM0;
  ra.snapM = F(lay.dMsnap_f);
  ra.Amat = rule == INFINI_RULE_DELTA ? F(lay.Amat_f) : nullptr;
  ra.reverse = 1;
  if ((d == dv ? infini::launch_chain(INFINI_F32, D, rule, ra, s)
               : infini::launch_chain_kv_f32(D, DV, rule, ra, s)) != hipSuccess)
    return INFINI_ERR_HIP;
  // dM_s^T in the element type for the update's products
  if (infini::launch_round_f32(dtype, E(lay.dMsnap), F(lay.dMsnap_f), units * S * d * dv, s) !=
      hipSuccess)
    return INFINI_ERR_HIP;

  // 4. local attention
  if (infini::launch_bwd_attention(dtype, D, DV, ba, s) != hipSuccess) return INFINI_ERR_HIP;

  // 5. update: dv_acc += sigma(K) dM_s, dphi, dc. bf16 with d in {64, 128}:
  // one fused kernel per 128 key rows, which writes dv = dv_acc + sigma(K)
  // dM_s as the output itself; otherwise key-side products (hi = unit) and a
  // row kernel.
  ba.dMsnap = E(lay.dMsnap);
  if (bwd_mfma) {
    ba.dv_final = 1;  // the kernel writes dv itself
    if (infini::launch_bwd_update_mfma(D, ba, s) != hipSuccess) return INFINI_ERR_HIP;
  } else {
    // key-side products, hi = unit: (rows of a d wide) x (M-shaped, stored
    // transposed [dv][d]) -> rows dv wide, or (rows dv wide) x (the stored
    // [dv][d] as is) -> rows d wide
    auto to_v = [&](const void* A, const void* Bm, float* C) {
      infini::GemmArgs g = gemm_args(A, Bm, C, N, DV, D, units, S, L, seg_len);
      g.lda = D;
      g.ldb = D;
      g.ldc = DV;
      g.a_hi = LD;
      g.a_lo = ND;
      g.c_hi = LV;
      g.c_lo = NV;
      g.b_hi = S * DDV;
      g.b_lo = DDV;
      g.tb = 1;
      g.a_sigma = 1;
      g.clip = 1;
      return g;
    };
    auto to_k = [&](const void* A, const void* Bm, float* C) {
      infini::GemmArgs g = gemm_args(A, Bm, C, N, D, DV, units, S, L, seg_len);
      g.lda = DV;
      g.ldb = D;
      g.ldc = D;
      g.a_hi = LV;
      g.a_lo = NV;
      g.c_hi = LD;
      g.c_lo = ND;
      g.b_hi = S * DDV;
      g.b_lo = DDV;
      g.tb = 0;
      g.clip = 1;
      return g;
    };
    {
      infini::GemmArgs g = to_v(k, E(lay.dMsnap), ba.du_buf);  // Phi dM_s (dM_s^T stored)
      if (infini::launch_gemm(dtype, g, s) != hipSuccess) return INFINI_ERR_HIP;
    }
    if (rule == INFINI_RULE_DELTA) {
      infini::GemmArgs g = to_v(k, E(lay.snapM), ba.p_buf);  // Phi M_{s-1}
      if (infini::launch_gemm(dtype, g, s) != hipSuccess) return INFINI_ERR_HIP;
    }
    if (infini::launch_bwd_update_rows(dtype, D, DV, ba, s) != hipSuccess) return INFINI_ERR_HIP;
    {  // (V - pred, or V) dM_s^T
      infini::GemmArgs g = to_k(rule == INFINI_RULE_DELTA ? ba.u_el : v, E(lay.dMsnap), ba.dphi);
      if (infini::launch_gemm(dtype, g, s) != hipSuccess) return INFINI_ERR_HIP;
    }
    if (rule == INFINI_RULE_DELTA) {
      infini::GemmArgs g = to_k(ba.dp_el, E(lay.snapM), ba.dphi);  // + dP M_{s-1}^T
      g.accumulate = 1;
      if (infini::launch_gemm(dtype, g, s) != hipSuccess) return INFINI_ERR_HIP;
    }
  }
  if (rule == INFINI_RULE_DELTA &&
      infini::launch_bwd_row_weighted_sum(dtype, D, DV, ba, false, s) != hipSuccess)
    return INFINI_ERR_HIP;

  // 6. dz, dK, dV, dbeta
  if (infini::launch_bwd_finish(dtype, D, DV, ba, s) != hipSuccess) return INFINI_ERR_HIP;
  return INFINI_OK;
}

}  // namespace

extern "C" {

infini_status_t infini_attn_backward(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d,
                                     int64_t seg_len, int32_t rule, int32_t dtype,
                                     const void* q, const void* k, const void* v,
                                     const float* beta, const float* M0, const float* z0,
                                     const void* out, const float* lse, const void* d_out,
                                     const float* dM_final, const float* dz_final, void* dq,
                                     void* dk, void* dv, float* dbeta, float* dM0, float* dz0,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(B, Hq, Hkv, L, d, d, seg_len, rule, dtype, q, k, v, beta, M0, z0, out, lse,
                       d_out, dM_final, dz_final, dq, dk, dv, dbeta, dM0, dz0, workspace,
                       workspace_bytes, stream);
}

infini_status_t infini_attn_backward_kv(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                        int64_t d_key, int64_t d_value, int64_t seg_len,
                                        int32_t rule, int32_t dtype, const void* q,
                                        const void* k, const void* v, const float* beta,
                                        const float* M0, const float* z0, const void* out,
                                        const float* lse, const void* d_out,
                                        const float* dM_final, const float* dz_final, void* dq,
                                        void* dk, void* dv, float* dbeta, float* dM0,
                                        float* dz0, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (d_value < 1) return INFINI_ERR_INVALID_ARG;
  return backward_impl(B, Hq, Hkv, L, d_key, d_value, seg_len, rule, dtype, q, k, v, beta, M0,
                       z0, out, lse, d_out, dM_final, dz_final, dq, dk, dv, dbeta, dM0, dz0,
                       workspace, workspace_bytes, stream);
}

// ---- the block with its projections -------------------------------------------

}  // extern "C"

namespace {

// Workspace of infini_attn_block_forward: q, k, v (head-major, bf16), the
// gated result a (head-major, bf16), then a full forward workspace.
struct BlockLayout {
  size_t q, k, v, a, fwd, fwd_bytes, total;
};

// d: the key width, dv: the value width ("Infini-Attention" (AI Wiki), "How
// does the compressive memory work?": M is d_key x d_value).
infini_status_t block_layout(int64_t B, int64_t L, int64_t d_model, int64_t Hq, int64_t Hkv,
                             int64_t d, int64_t dv, int64_t seg_len, int32_t rule,
                             int32_t dtype, BlockLayout* lay) {
  Plan p;
  infini_status_t st = check_sizes_kv(B, Hq, Hkv, L, d, dv, seg_len, rule, dtype, &p);
  if (st != INFINI_OK) return st;
  if (d_model < 1) return INFINI_ERR_INVALID_ARG;
  if (dtype != INFINI_BF16) return INFINI_ERR_UNSUPPORTED;  // the projections are bf16 MFMA
  if (d_model % 32 != 0) return INFINI_ERR_UNSUPPORTED;     // K steps of 32
  // 32-bit row and column indices in the projection kernel, 32-bit lane
  // offsets within its loads (rows of one 256-row tile)
  const int64_t M = B * L, Nqkv = (Hq + Hkv) * d + Hkv * dv;
  if (M >= INT32_MAX || Nqkv >= INT32_MAX || d_model >= (1 << 22)) return INFINI_ERR_INVALID_ARG;
  if ((256 * Hq + Hq * L + L) * dv * 2 >= (int64_t)UINT32_MAX) return INFINI_ERR_INVALID_ARG;
  const int64_t tiles = ((M + 255) / 256) * (((Nqkv > d_model ? Nqkv : d_model) + 255) / 256);
  if (tiles > INT32_MAX) return INFINI_ERR_INVALID_ARG;
  if (lay) {
    const size_t nq = align_up((size_t)(B * Hq * L * d) * 2);
    const size_t nk = align_up((size_t)(B * Hkv * L * d) * 2);
    const size_t nv = align_up((size_t)(B * Hkv * L * dv) * 2);
    const size_t na = align_up((size_t)(B * Hq * L * dv) * 2);
    lay->q = 0;
    lay->k = nq;
    lay->v = nq + nk;
    lay->a = nq + nk + nv;
    lay->fwd = nq + nk + nv + na;
    lay->fwd_bytes = workspace_full(p);
    lay->total = lay->fwd + lay->fwd_bytes;
  }
  return INFINI_OK;
}

infini_status_t block_impl(int64_t B, int64_t L, int64_t d_model, int64_t Hq, int64_t Hkv,
                           int64_t d, int64_t dv, int64_t seg_len, int32_t rule,
                           int32_t dtype, const void* x, const void* w_qkv, const void* w_o,
                           const float* beta, const float* M0, const float* z0, void* y,
                           float* M_final, float* z_final, void* workspace,
                           size_t workspace_bytes, void* stream, void* const* events,
                           int32_t n_events) {
  BlockLayout lay;
  infini_status_t st =
      block_layout(B, L, d_model, Hq, Hkv, d, dv, seg_len, rule, dtype, &lay);
  if (st != INFINI_OK) return st;
  const void* ptrs[] = {x, w_qkv, w_o, beta, M0, z0, y, M_final, z_final, workspace};
  for (const void* ptr : ptrs)
    if (ptr == nullptr) return INFINI_ERR_INVALID_ARG;
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return INFINI_ERR_MISALIGNED;
  if (workspace_bytes < lay.total) return INFINI_ERR_WORKSPACE;
  if (n_events < 0 || (n_events > 0 && events == nullptr)) return INFINI_ERR_INVALID_ARG;
  for (int32_t e = 0; e < n_events; ++e)
    if (events[e] == nullptr) return INFINI_ERR_INVALID_ARG;

  const int64_t M = B * L, Nqkv = (Hq + Hkv) * d + Hkv * dv;
  const size_t nx = (size_t)(M * d_model) * 2, ny = nx;
  const size_t nwq = (size_t)(Nqkv * d_model) * 2, nwo = (size_t)(d_model * Hq * dv) * 2;
  const size_t nM = (size_t)(B * Hkv * d * dv) * 4, nz = (size_t)(B * Hkv * d) * 4;
  struct Range { const void* p; size_t n; };
  const Range inputs[] = {{x, nx}, {w_qkv, nwq}, {w_o, nwo}, {beta, (size_t)Hq * 4},
                          {M0, nM}, {z0, nz}};
  // y and the workspace overlap nothing; M_final / z_final may coincide
  // exactly with M0 / z0 (the forward checks those among themselves)
  for (const Range& r : inputs) {
    if (overlap(y, ny, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (overlap(workspace, workspace_bytes, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (r.p != M0 && overlap(M_final, nM, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
    if (r.p != z0 && overlap(z_final, nz, r.p, r.n)) return INFINI_ERR_INVALID_ARG;
  }
  if (overlap(y, ny, workspace, workspace_bytes) || overlap(y, ny, M_final, nM) ||
      overlap(y, ny, z_final, nz) || overlap(workspace, workspace_bytes, M_final, nM) ||
      overlap(workspace, workspace_bytes, z_final, nz))
    return INFINI_ERR_INVALID_ARG;

  char* ws = static_cast<char*>(workspace);
  void* q = ws + lay.q;
  void* k = ws + lay.k;
  void* v = ws + lay.v;
  void* a = ws + lay.a;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int slot) -> bool {
    if (slot >= n_events) return true;
    return hipEventRecord(static_cast<hipEvent_t>(events[slot]), s) == hipSuccess;
  };

  // 1. q, k, v = x W_qkv^T, split into heads
  infini::ProjArgs pa{};
  pa.a = x;
  pa.w = w_qkv;
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.M = M;
  pa.N = Nqkv;
  pa.K = d_model;
  pa.lda = d_model;
  pa.a_elems = M * d_model;
  pa.L = L;
  pa.d = d;
  pa.dv = dv;
  pa.Ha = 1;
  pa.Hq = Hq;
  pa.Hkv = Hkv;
  pa.a_mode = infini::kProjRows;
  pa.c_mode = infini::kProjHeads;
  if (!mark(0)) return INFINI_ERR_HIP;
  if (infini::launch_proj(pa, s) != hipSuccess) return INFINI_ERR_HIP;
  if (!mark(1)) return INFINI_ERR_HIP;

  // 2. the block: a, M_final, z_final
  st = forward_impl(B, Hq, Hkv, L, d, seg_len, rule, dtype, q, k, v, beta, M0, z0, a, M_final,
                    z_final, nullptr, ws + lay.fwd, lay.fwd_bytes, stream, nullptr, 0, dv);
  if (st != INFINI_OK) return st;
  if (!mark(2)) return INFINI_ERR_HIP;

  // 3. y = concat_h(a_h) W_o^T, a read in place (head-major)
  infini::ProjArgs po{};
  po.a = a;
  po.w = w_o;
  po.c = y;
  po.M = M;
  po.N = d_model;
  po.K = Hq * dv;
  po.ldc = d_model;
  po.a_elems = B * Hq * L * dv;
  po.L = L;
  po.d = dv;  // a's heads are d_value wide
  po.dv = dv;
  po.Ha = Hq;
  po.Hq = Hq;
  po.Hkv = Hkv;
  po.a_mode = infini::kProjGather;
  po.c_mode = infini::kProjRows;
  if (infini::launch_proj(po, s) != hipSuccess) return INFINI_ERR_HIP;
  if (!mark(3)) return INFINI_ERR_HIP;
  return INFINI_OK;
}

}  // namespace

extern "C" {

infini_status_t infini_attn_block_workspace_size(int64_t B, int64_t L, int64_t d_model,
                                                 int64_t Hq, int64_t Hkv, int64_t d,
                                                 int64_t seg_len, int32_t rule, int32_t dtype,
                                                 size_t* bytes) {
  if (bytes == nullptr) return INFINI_ERR_INVALID_ARG;
  BlockLayout lay;
  const infini_status_t st =
      block_layout(B, L, d_model, Hq, Hkv, d, d, seg_len, rule, dtype, &lay);
  if (st != INFINI_OK) return st;
  *bytes = lay.total;
  return INFINI_OK;
}

infini_status_t infini_attn_block_forward(int64_t B, int64_t L, int64_t d_model, int64_t Hq,
                                          int64_t Hkv, int64_t d, int64_t seg_len,
                                          int32_t rule, int32_t dtype, const void* x,
                                          const void* w_qkv, const void* w_o, const float* beta,
                                          const float* M0, const float* z0, void* y,
                                          float* M_final, float* z_final, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return block_impl(B, L, d_model, Hq, Hkv, d, d, seg_len, rule, dtype, x, w_qkv, w_o, beta,
                    M0, z0, y, M_final, z_final, workspace, workspace_bytes, stream, nullptr, 0);
}

infini_status_t infini_attn_block_workspace_size_kv(int64_t B, int64_t L, int64_t d_model,
                                                    int64_t Hq, int64_t Hkv, int64_t d_key,
                                                    int64_t d_value, int64_t seg_len,
                                                    int32_t rule, int32_t dtype, size_t* bytes) {
  if (bytes == nullptr || d_value < 1) return INFINI_ERR_INVALID_ARG;
  BlockLayout lay;
  const infini_status_t st =
      block_layout(B, L, d_model, Hq, Hkv, d_key, d_value, seg_len, rule, dtype, &lay);
  if (st != INFINI_OK) return st;
  *bytes = lay.total;
  return INFINI_OK;
}

infini_status_t infini_attn_block_forward_kv(int64_t B, int64_t L, int64_t d_model, int64_t Hq,
                                             int64_t Hkv, int64_t d_key, int64_t d_value,
                                             int64_t seg_len, int32_t rule, int32_t dtype,
                                             const void* x, const void* w_qkv, const void* w_o,
                                             const float* beta, const float* M0,
                                             const float* z0, void* y, float* M_final,
                                             float* z_final, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  if (d_value < 1) return INFINI_ERR_INVALID_ARG;
  return block_impl(B, L, d_model, Hq, Hkv, d_key, d_value, seg_len, rule, dtype, x, w_qkv, w_o,
                    beta, M0, z0, y, M_final, z_final, workspace, workspace_bytes, stream,
                    nullptr, 0);
}

infini_status_t infini_attn_block_forward_timed(
    int64_t B, int64_t L, int64_t d_model, int64_t Hq, int64_t Hkv, int64_t d, int64_t seg_len,
    int32_t rule, int32_t dtype, const void* x, const void* w_qkv, const void* w_o,
    const float* beta, const float* M0, const float* z0, void* y, float* M_final,
    float* z_final, void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events) {
  return block_impl(B, L, d_model, Hq, Hkv, d, d, seg_len, rule, dtype, x, w_qkv, w_o, beta,
                    M0, z0, y, M_final, z_final, workspace, workspace_bytes, stream, events,
                    n_events);
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

const char* infini_attn_error_string(int32_t status) { return infini_attn_status_string(status); }

int32_t infini_attn_version(void) { return kVersion; }

}  // extern "C"
