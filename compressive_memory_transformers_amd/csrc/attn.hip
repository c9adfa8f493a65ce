// Local causal attention with the memory retrieval and the gate fused in.
//
// "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
// block?": A_dot = causal softmax(Q K^T / sqrt(d)) V inside the segment,
// A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1}), and
// out = sigmoid(beta) A_mem + (1 - sigmoid(beta)) A_dot.
//
// One workgroup computes 32*NW query rows of one (batch, query head, segment);
// every segment of a window runs in parallel, because the only thing a segment
// needs from its predecessors is the state snapshot the scan wrote.
//
// Each wave owns 32 query rows and forms S^T = K Q^T rather than Q K^T: in the
// 32x32 accumulator a lane then holds one query (its column) and 16 keys, so a
// query's running max and sum need only one exchange between the two
// half-waves, and the probabilities sit in registers exactly where the B
// operand of O^T += V^T P^T wants them (keys in the accumulator's row order).
// Q stays in registers for the whole key loop; K tiles are staged in LDS row
// major, V tiles transposed, so every MFMA operand is a 16- or 8-byte LDS read.
//
// The retrieval reuses the output accumulator: after the key loop the
// accumulator is scaled by (1 - g)/l per query, and one more product
// O^T += M^T (g sigma(Q) / den)^T adds the gated memory read, with the
// per-query factor g/den folded into the B operand.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace infini {

namespace {

// Threshold of the lazy softmax rescale, in log2 units: the running max a
// query's exponents are taken against is only raised when a new score exceeds
// it by more than this, so exp2 arguments stay <= kRescaleTau and the
// accumulator is rescaled rarely. The result is exact either way: numerator
// and denominator use the same reference.
constexpr float kRescaleTau = 8.f;
constexpr float kRescaleBound = 256.f;  // 2^kRescaleTau

// DK: the key width (Q, K, rows of M); DV: the value width (V, the output,
// columns of M).
template <typename T, int DK, int DV, int NW, int BN>
struct AttnTile {
  static constexpr int NT = NW * 64;
  // Row strides (elements). K rows: 16 bytes of padding, so the 16 lanes of a
  // quarter-wave reading 16-byte chunks of 16 consecutive rows hit 16
  // different 4-bank groups. V^T rows: 4 elements of padding, so 32 lanes
  // reading 4-element runs of 32 consecutive rows, and the transposed stores
  // below, each cover the 64 banks once.
  static constexpr int KS = DK + pad16<T>();
  static constexpr int VS = BN + 4;
  static constexpr int K_TOTAL = BN * (DK / 8);  // 8-element K chunks per tile
  static constexpr int K_CHUNKS = (K_TOTAL + NT - 1) / NT;  // per thread
  // V is staged in 4 keys x 4 dims blocks; a group of 32 lanes takes 8
  // consecutive dim-quads x 4 consecutive key-quads.
  static constexpr int DQ = DV / 4, KQ = BN / 4;
  static constexpr int V_GROUPS = (DQ / 8) * (KQ / 4);
  static constexpr int V_PER_THREAD = (V_GROUPS * 32 + NT - 1) / NT;
  static_assert(DQ % 8 == 0 && KQ % 4 == 0, "V staging layout");
  frag_t<T> k[K_CHUNKS];
  vec4_t<T> v[V_PER_THREAD][4];

  __device__ __forceinline__ static bool k_item(int j, int tid, int& r, int& col) {
    const int c = tid + j * NT;
    r = c / (DK / 8);
    col = (c % (DK / 8)) * 8;
    return K_TOTAL % NT == 0 || c < K_TOTAL;
  }
  __device__ __forceinline__ static bool v_item(int j, int tid, int& d4, int& k4) {
    const int g = (tid >> 5) + j * (NT / 32), l = tid & 31;
    d4 = (g % (DQ / 8)) * 8 + (l & 7);
    k4 = (g / (DQ / 8)) * 4 + (l >> 3);
    return (V_GROUPS * 32) % NT == 0 || g < V_GROUPS;
  }

  // Global -> registers for key tile k0. Rows past the segment's end repeat
  // its last row: finite values whose scores the causal mask removes.
  __device__ __forceinline__ void load(const T* K, const T* V, int k0, int n_s, int tid) {
    const int last = n_s - 1;
#pragma unroll
    for (int j = 0; j < K_CHUNKS; ++j) {
      int r, col;
      if (k_item(j, tid, r, col)) k[j] = load8<T>(K + (int64_t)min(k0 + r, last) * DK + col);
    }
#pragma unroll
    for (int j = 0; j < V_PER_THREAD; ++j) {
      int d4, k4;
      if (v_item(j, tid, d4, k4)) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[j][q] = load4<T>(V + (int64_t)min(k0 + 4 * k4 + q, last) * DV + 4 * d4);
      }
    }
  }

  // Registers -> LDS: K row major, V transposed.
  __device__ __forceinline__ void store(T* Ks, T* Vt, int tid) const {
#pragma unroll
    for (int j = 0; j < K_CHUNKS; ++j) {
      int r, col;
      if (k_item(j, tid, r, col)) store8<T>(Ks + r * KS + col, k[j]);
    }
#pragma unroll
    for (int j = 0; j < V_PER_THREAD; ++j) {
      int d4, k4;
      if (v_item(j, tid, d4, k4)) {
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          vec4_t<T> y;
          y[0] = v[j][0][dd]; y[1] = v[j][1][dd]; y[2] = v[j][2][dd]; y[3] = v[j][3][dd];
          store4<T>(Vt + (4 * d4 + dd) * VS + 4 * k4, y);
        }
      }
    }
  }
};

// One key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// MASK: the tile reaches past the wave's first query row, so the causal mask
// applies (only the tiles on the diagonal).
template <typename T, int DK, int DV, int BN, bool MASK>
__device__ __forceinline__ void attn_tile(const T* Kb, const T* Vb, const frag_t<T>* qf,
                                          f32x16* oacc, float& m_run, float& l_run, float c,
                                          int k0, int row, int i, int h) {
  constexpr int NC = DK / 16, NDB = DV / 32, NKB = BN / 32, NPC = BN / 16;
  constexpr int KS = DK + pad16<T>();
  constexpr int VS = BN + 4;
  f32x16 sacc[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    sacc[kb] = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      mma32(sacc[kb], load8<T>(Kb + (32 * kb + i) * KS + 16 * cc + 8 * h), qf[cc]);
  }
  if constexpr (MASK) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (k0 + 32 * kb + acc_row(r, h) > row) sacc[kb][r] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
  mx = xhalf_max(mx);
  // Key 0 of the segment is visible to every row, so the first tile sets a
  // finite reference for every lane.
  if (__any((mx - m_run) * c > kRescaleTau)) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    m_run = m_new;
  }
  const float mc = m_run * c;
  frag_t<T> pf[NPC];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c, -mc));
      l_run += p;
      pf[2 * kb + (r >> 3)][r & 7] = from_f32<T>(p);
    }
  // O^T += V^T P^T. Element e of pf[pc] is key 16pc + 8(e/4) + 4h + e%4 of the
  // tile, so the A operand reads two runs of four keys from Vt.
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) {
      const T* vrow = Vb + (32 * db + i) * VS + 16 * pc + 4 * h;
      mma32(oacc[db], load4x2<T>(vrow, vrow + 8), pf[pc]);
    }
}

template <typename T, int DK, int DV, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 2) void attn_kernel(AttnArgs a) {
  using Tile = AttnTile<T, DK, DV, NW, BN>;
  constexpr int BM = 32 * NW;
  constexpr int NC = DK / 16;   // 16-wide chunks of the key dimension
  constexpr int NDB = DV / 32;  // 32-row blocks of the value dimension
  constexpr int NKB = BN / 32;  // 32-key blocks of a key tile
  constexpr int NPC = BN / 16;  // 16-key chunks of a key tile
  constexpr int KS = Tile::KS;
  constexpr int VS = Tile::VS;

  // Two buffers: tile kt+1 is written while tile kt is read.
  __shared__ __align__(16) T Ks[2][BN * KS];  // K tiles, [key][dim]
  __shared__ __align__(16) T Vt[2][DV * VS];  // V tiles transposed, [dim][key]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 31, h = lane >> 5;

  // Tile order. Hardware hands consecutive workgroups to the 8 XCDs in turn;
  // remapping makes each XCD take a contiguous range of logical tiles, so the
  // query tiles and grouped heads that read one segment's K/V share an L2.
  // Within a (batch, KV head, segment) group the heaviest query tiles (the
  // longest causal rows) come first.
  int t = blockIdx.x;
  {
    const int per = (int)(gridDim.x >> 3);
    if (t < per * 8) t = (t & 7) * per + (t >> 3);
  }
  const int G = a.Hq / a.Hkv;
  const int in_grp = a.n_qt * G;
  const int grp = t / in_grp, rr = t % in_grp;
  const int qt = a.n_qt - 1 - rr / G;
  const int hg = rr % G;
  const int sl = grp % a.s_count;
  const int unit = grp / a.s_count;  // b * Hkv + kv head
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int hq = kvh * G + hg;
  const int64_t seg_start = (int64_t)(a.s_begin + sl) * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  const int q0 = qt * BM;
  if (q0 >= n_s) return;  // the tail of a short last segment; uniform per workgroup

  const int64_t qh = (int64_t)b * a.Hq + hq;
  const T* Q = static_cast<const T*>(a.q) + (qh * a.L + seg_start) * DK;
  const T* K = static_cast<const T*>(a.k) + ((int64_t)unit * a.L + seg_start) * DK;
  const T* V = static_cast<const T*>(a.v) + ((int64_t)unit * a.L + seg_start) * DV;
  T* O = static_cast<T*>(a.out) + (qh * a.L + seg_start) * DV;

  const int row = q0 + 32 * w + i;  // this lane's query, relative to the segment
  const bool wave_on = q0 + 32 * w < n_s;
  const int wave_last = min(q0 + 32 * w + 31, n_s - 1);
  const float c = a.scale_log2;

  const int n_kv = min(q0 + BM, n_s);  // keys any row of the workgroup can see
  const int n_kt = (n_kv + BN - 1) / BN;

  Tile tile;
  tile.load(K, V, 0, n_s, tid);

  // B operand of S^T = K Q^T: column i is query `row`, k = 16c + 8h + e.
  frag_t<T> qf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    qf[cc] = zero_frag<T>();
    if (row < n_s) qf[cc] = load8<T>(Q + (int64_t)row * DK + 16 * cc + 8 * h);
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero16();
  float m_run = -INFINITY;  // reference max of this query's raw scores
  float l_run = 0.f;        // this half-wave's share of the softmax sum

  tile.store(Ks[0], Vt[0], tid);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BN;
    const int buf = kt & 1;
    if (kt + 1 < n_kt) tile.load(K, V, k0 + BN, n_s, tid);  // in flight during this tile

    if (wave_on && k0 <= wave_last) {
      if (k0 + BN - 1 > q0 + 32 * w)
        attn_tile<T, DK, DV, BN, true>(Ks[buf], Vt[buf], qf, oacc, m_run, l_run, c, k0, row, i, h);
      else
        attn_tile<T, DK, DV, BN, false>(Ks[buf], Vt[buf], qf, oacc, m_run, l_run, c, k0, row, i,
                                        h);
    }
    if (kt + 1 < n_kt) {
      // buffer buf^1 was last read in iteration kt-1, before that iteration's
      // barrier
      tile.store(Ks[buf ^ 1], Vt[buf ^ 1], tid);
      __syncthreads();
    }
  }
  if (!wave_on) return;  // no barrier follows

  const float l = xhalf_sum(l_run);
  if (a.lse != nullptr && h == 0 && row < n_s)
    a.lse[qh * a.L + seg_start + row] = m_run * c + __log2f(l);
  const int64_t snap = (int64_t)unit * a.snap_count + a.snap_first + sl;
  const float* zs = a.snapZ + snap * DK;
  const T* Mts = static_cast<const T*>(a.snapM) + snap * DV * DK;

  float sq[NC][8];
  float dp = 0.f;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = feature_map(to_f32<T>(qf[cc][e]));
      sq[cc][e] = s;
      dp += s * zs[16 * cc + 8 * h + e];
    }
  const float den = xhalf_sum(dp);
  const float g = 1.f / (1.f + __expf(-a.beta[hq]));
  const float ca = (1.f - g) / l, cm = g / den;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] *= ca;
  frag_t<T> sf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) sf[cc][e] = from_f32<T>(sq[cc][e] * cm);
  // O^T += M^T (g sigma(Q)/den)^T; the snapshot is M^T, [value][key].
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      mma32(oacc[db], load8<T>(Mts + (int64_t)(32 * db + i) * DK + 16 * cc + 8 * h), sf[cc]);

  if (row < n_s) {
    T* orow = O + (int64_t)row * DV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        vec4_t<T> y;
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = from_f32<T>(oacc[db][4 * rq + j]);
        store4<T>(orow + 32 * db + 8 * rq + 4 * h, y);
      }
  }
}

// ---- bf16, d in {64, 128}: tiles streamed straight into LDS ------------------
//
// K and V tiles go from global memory into LDS by DMA (DmaTile, lds_tile.hpp),
// row major with XOR-swizzled 16-byte chunks; K is read as the A operand of
// S^T = K Q^T with 16-byte reads, V as the A operand of O^T += V^T P^T with
// transposing reads.

// Per-lane state of the key loop, with the lane's LDS read offsets computed
// once: with the swizzles above, a lane's K and V read addresses differ
// between key blocks, probability chunks and the two LDS buffers only by
// constants, which the reads take as immediate offsets.
template <int DK, int DV>
struct DmaLane {
  static constexpr int NC = DK / 16, NDB = DV / 32;
  bf16x8 qf[NC];
  f32x16 oacc[NDB];
  float m_run, l0, l1;  // running max (log2 units before scaling) and two partial sums
  uint32_t ko;          // K: byte offset of chunk h of tile row i; chunk 2cc + h is at ko ^ 32cc
  uint32_t vo[NDB];     // V: byte offset of this lane's transposing read for value block db

  __device__ __forceinline__ void init_offsets(int lane) {
    const int i = lane & 31, h = lane >> 5;
    ko = 2 * (i * DK + 8 * (h ^ swz_k<DK>(i)));
#pragma unroll
    for (int db = 0; db < NDB; ++db) vo[db] = tr_offset<DV>(lane, db);
  }
};

// The key loop is software-pipelined by one tile, so that each wave has
// matrix work to issue beside its softmax arithmetic: iteration j issues
// S(j+1) = K(j+1) Q^T and O += V(j) P(j) (P(j) formed in the iteration
// before) back to back on the matrix cores, then forms P(j+1) from S(j+1)
// while O's products run.

// S^T = K Q^T for one key tile (K in LDS).
template <int DK, int DV, int BN>
__device__ __forceinline__ void dma_scores(const bf16* Kb, const DmaLane<DK, DV>& st,
                                           f32x16* sacc) {
  constexpr int NC = DK / 16, NKB = BN / 32;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    sacc[kb] = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      mma32(sacc[kb], load8<bf16>(lds_at(Kb, (st.ko ^ (32u * cc)) + 2 * 32 * kb * DK)), st.qf[cc]);
  }
}

// Causal mask (on a tile that crosses the wave's diagonal), then the
// probabilities exp2(c s - c m) of the tile against the running maximum m as
// the bf16 B operand of O^T += V^T P^T, with their row sums as rounded for
// that product (pairwise, v_dot2_f32_bf16 against (1, 1)). The lazy rescale
// is decided from the sums: each lane's sum over its 32 probabilities of the
// tile bounds every one of them, so while no lane's sum exceeds
// 2^kRescaleTau (and none is not a number, as with the first tile's
// m = -inf) no probability does, and the stale m stands. Otherwise (rarely)
// the wave takes the tile's row maxima, rescales O and l, and forms the
// probabilities again. No row maximum is taken on the common path.
template <int DK, int DV, int BN>
__device__ __forceinline__ void dma_probs_lazy(f32x16* s, DmaLane<DK, DV>& st, float c, int k0,
                                               int row, int h, bool diag, bf16x8* pf) {
  constexpr int NDB = DV / 32, NKB = BN / 32, NPC = BN / 16;
  if (diag) {  // wave-uniform
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (k0 + 32 * kb + acc_row(r, h) > row) s[kb][r] = -INFINITY;
  }
  float t0, t1;
  auto form = [&]() {
    const float mc = st.m_run * c;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pf[2 * kb + (r >> 3)][r & 7] = (bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
    t0 = t1 = 0.f;
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 pr = {pf[pc][2 * q], pf[pc][2 * q + 1]};
        if (q & 1)
          t1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, t1, false);
        else
          t0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, t0, false);
      }
  };
  form();
  if (__any(!(t0 + t1 <= kRescaleBound))) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xhalf_max(mx);
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((st.m_run - m_new) * c);
    st.l0 *= alpha;
    st.l1 *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
    st.m_run = m_new;
    form();
  }
  st.l0 += t0;
  st.l1 += t1;
}

// O^T += V^T P^T for one key tile (V in LDS, read transposed).
template <int DK, int DV, int BN>
__device__ __forceinline__ void dma_values(const bf16* Vb, DmaLane<DK, DV>& st,
                                           const bf16x8* pf) {
  constexpr int NDB = DV / 32, NPC = BN / 16;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) mma32(st.oacc[db], tr_frag<DV>(Vb, st.vo[db], pc), pf[pc]);
}

// The retrieval's operands, loaded during the workgroup's last key tile into
// the two LDS buffers that tile no longer needs: M^T (d x d, element type)
// rows 0..63 into Ma and rows 64..127 (d = 128) into Mb, with the K tile
// layout, so the epilogue reads its A operand as it reads K; z (d floats)
// into Zs by one 16-byte load per lane of wave 0 (lanes past d/4 read
// outside the resource, which returns zeros).
template <int DK, int DV, int NW, int BN>
__device__ __forceinline__ void dma_snapshot(const DmaTile<DK, NW, BN>& tile, const bf16* Mts,
                                             const float* zs, bf16* Ma, bf16* Mb, float* Zs,
                                             int w) {
  // M^T is d_value rows of d_key: d_value / 64 tiles in the K layout; the
  // second goes to a V buffer, at least as large when d_value = 128
  static_assert(BN == 64 && DV % 64 == 0, "M^T is loaded as d_value / 64 key tiles");
  tile.template issue<true>(Mts, Ma, 0, 64, w);
  if constexpr (DV == 128) tile.template issue<true>(Mts + 64 * DK, Mb, 0, 64, w);
  if (w == 0) {
    const __amdgpu_buffer_rsrc_t rz = raw_rsrc(reinterpret_cast<const bf16*>(zs), DK * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_void*)Zs, 16, (threadIdx.x & 63) * 16, 0, 0, 0);
  }
}

// Iteration j of the key loop on LDS buffer parity P = j % 2 (a constant, so
// every LDS address is a lane offset plus an immediate). On entry K(j + 1) is
// in Ks[P ^ 1] and V(j) in Vs[P]; pf holds the probabilities of tile j.
// The iteration loads K(j + 2) over K(j) and V(j + 1) over V(j - 1), both
// last read before the previous barrier, and waits for them at its end.
// FULL: the caller knows that tile j + 1 is this wave's too and below its
// diagonal (every iteration but a workgroup's last few), so tile j + 2
// exists and the iteration is one straight-line block apart from the rare
// rescale. The loads and the wait are then unconditional, which lets the
// compiler see that the reads of this iteration touch only the other two
// buffers (separate arrays) and need not wait for the loads just issued.
template <int DK, int DV, int NW, int BN, int P, bool FULL>
__device__ __forceinline__ void dma_iter(int j, int n_kt, int n_w,
                                         const DmaTile<DK, NW, BN>& tile,
                                         const DmaTile<DV, NW, BN>& vtile, const bf16* K,
                                         const bf16* V, bf16* const* Ks, bf16* const* Vs, int n_s,
                                         int w, int wfirst, DmaLane<DK, DV>& st, bf16x8* pf,
                                         float c, int row, int h, const bf16* Mts,
                                         const float* zs, float* Zs) {
  constexpr int NKB = BN / 32, NPC = BN / 16;
  if (FULL) {
    tile.template issue_full<true>(K, Ks[P], (j + 2) * BN, w);
    vtile.template issue_full<false>(V, Vs[P ^ 1], (j + 1) * BN, w);
  } else {
    if (j + 2 < n_kt) tile.template issue<true>(K, Ks[P], (j + 2) * BN, n_s, w);
    if (j + 1 < n_kt) vtile.template issue<false>(V, Vs[P ^ 1], (j + 1) * BN, n_s, w);
  }
  if (!FULL && j + 1 == n_kt)
    dma_snapshot<DK, DV, NW, BN>(tile, Mts, zs, Ks[P], Vs[P ^ 1], Zs, w);
  if (FULL || j + 1 < n_w) {
    f32x16 snext[NKB];
    dma_scores<DK, DV, BN>(Ks[P ^ 1], st, snext);
    dma_values<DK, DV, BN>(Vs[P], st, pf);
    // the scheduler's strategy that interleaves LDS reads with the matrix
    // products: 1.3% faster on the full iterations (alternating A/B timing;
    // the strategies for other instruction mixes were slower)
    if constexpr (FULL) __builtin_amdgcn_iglp_opt(0);
    const int k1 = (j + 1) * BN;
    dma_probs_lazy<DK, DV, BN>(snext, st, c, k1, row, h, !FULL && k1 + BN - 1 > wfirst, pf);
  } else if (!FULL && j < n_w) {  // this wave's last tile
    dma_values<DK, DV, BN>(Vs[P], st, pf);
  }
  if (FULL || j + 1 < n_kt) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of K(j + 2), V(j + 1) have landed
    __syncthreads();
  }
}

// DK: the key width (Q, K); DV: the value width (V, the output).
// PACK (NW query heads of one KV head per workgroup, the group size a
// multiple of NW): wave w takes 32 consecutive positions of the group's head
// w (lane i: position q0 + i), so the four waves share one causal diagonal,
// 32 keys wide, where 128 rows of one head span 128 keys. At 2048-token
// segments a block then runs 16.5 64-key tiles on average instead of 17, and
// the tiles it masks drop from two to one. The K and V tiles, M^T and z are
// the KV head's, shared by the four heads as they are by four one-head
// blocks.
template <int DK, int DV, int NW, int BN, bool PACK>
__global__ __launch_bounds__(NW * 64, 2) void attn_kernel_dma(AttnArgs a) {
  constexpr int BM = PACK ? 32 : 32 * NW;  // positions per block
  constexpr int NC = DK / 16, NDB = DV / 32;
  // four separate arrays, so that the compiler can tell a tile being loaded
  // by DMA from the tiles being read and does not wait for the load
  __shared__ __align__(1024) bf16 Ks0[BN * DK];
  __shared__ __align__(1024) bf16 Ks1[BN * DK];
  __shared__ __align__(1024) bf16 Vs0[BN * DV];
  __shared__ __align__(1024) bf16 Vs1[BN * DV];
  bf16* const Ks[2] = {Ks0, Ks1};
  bf16* const Vs[2] = {Vs0, Vs1};
  __shared__ __align__(16) float Zs[256];  // z of the segment (one 16-byte DMA per lane of wave 0)

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;

  int t = blockIdx.x;
  {
    const int per = (int)(gridDim.x >> 3);
    if (t < per * 8) t = (t & 7) * per + (t >> 3);
  }
  const int G = a.Hq / a.Hkv;
  // n_qt G blocks per (unit, segment), heaviest first: n_qt query tiles of
  // 32 NW rows times G heads, or (PACK) NW n_qt position blocks of 32 times
  // G / NW head groups; blocks past the segment's end return at once
  const int in_grp = a.n_qt * G;
  const int grp = t / in_grp, rr = t % in_grp;
  int q0, hg;
  if constexpr (PACK) {
    const int n_sub = G / NW;
    q0 = (a.n_qt * NW - 1 - rr / n_sub) * BM;
    hg = (rr % n_sub) * NW + w;
  } else {
    q0 = (a.n_qt - 1 - rr / G) * BM;
    hg = rr % G;
  }
  const int sl = grp % a.s_count;
  const int unit = grp / a.s_count;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int hq = kvh * G + hg;
  const int64_t seg_start = (int64_t)(a.s_begin + sl) * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  if (q0 >= n_s) return;

  const int64_t qh = (int64_t)b * a.Hq + hq;
  const bf16* Q = static_cast<const bf16*>(a.q) + (qh * a.L + seg_start) * DK;
  const bf16* K = static_cast<const bf16*>(a.k) + ((int64_t)unit * a.L + seg_start) * DK;
  const bf16* V = static_cast<const bf16*>(a.v) + ((int64_t)unit * a.L + seg_start) * DV;

  // Without PACK the rows are dealt to the waves round robin (row q0 + w +
  // NW i for lane i), so every wave spans the whole block and meets the
  // causal diagonal in the same key tiles: the waves run the same number of
  // iterations and none idles at the barriers of the block's last tiles.
  // With PACK every wave holds the same 32 positions (of its own head).
  const int row = PACK ? q0 + i : q0 + w + NW * i;  // this lane's query, relative to the segment
  int wave_first = PACK ? q0 : q0 + w;
  // Opaque to the optimiser: with PACK, knowing wave_first == q0 (so every
  // wave active) led it to keep about 32 more registers live through the key
  // loop, which spilled at d = 128.
  asm volatile("" : "+s"(wave_first));
  const bool wave_on = wave_first < n_s;
  const int wave_last = !wave_on ? -1
                        : PACK   ? min(q0 + 31, n_s - 1)
                                 : wave_first + NW * min(31, (n_s - 1 - wave_first) / NW);
  const float c = a.scale_log2;
  const int n_kv = min(q0 + BM, n_s);
  const int n_kt = (n_kv + BN - 1) / BN;

  DmaTile<DK, NW, BN> tile;  // K tiles (and M^T), rows of d_key
  tile.init(w, lane);
  DmaTile<DV, NW, BN> vtile;  // V tiles, rows of d_value
  vtile.init(w, lane);
  tile.template issue<true>(K, Ks[0], 0, n_s, w);
  vtile.template issue<false>(V, Vs[0], 0, n_s, w);
  if (n_kt > 1) tile.template issue<true>(K, Ks[1], BN, n_s, w);

  DmaLane<DK, DV> st;
  st.init_offsets(lane);
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    st.qf[cc] = zero_frag<bf16>();
    if (row < n_s) st.qf[cc] = load8<bf16>(Q + (int64_t)row * DK + 16 * cc + 8 * h);
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db) st.oacc[db] = zero16();
  st.m_run = -INFINITY;
  st.l0 = st.l1 = 0.f;

  // key tiles this wave computes (its last is the one holding its last row)
  const int n_w = wave_on ? wave_last / BN + 1 : 0;
  constexpr int NKB = BN / 32, NPC = BN / 16;
  bf16x8 pf[NPC];  // the probabilities of the next tile to multiply into O
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n_w > 0) {
    f32x16 s0[NKB];
    dma_scores<DK, DV, BN>(Ks[0], st, s0);
    dma_probs_lazy<DK, DV, BN>(s0, st, c, 0, row, h, BN - 1 > wave_first, pf);
  }
  __syncthreads();  // K(0) read by every wave before iteration 0 loads K(2) over it
  // When every row of the block is in the segment, iterations j whose next
  // tile j + 1 lies wholly below the block's first row are full for every
  // wave.
  const int n_full = q0 + BM <= n_s ? min(q0 / BN - 1, n_s / BN - 2) : 0;
  const int64_t snap = (int64_t)unit * a.snap_count + a.snap_first + sl;
  const float* zs = a.snapZ + snap * DK;
  const bf16* Mts = static_cast<const bf16*>(a.snapM) + snap * DV * DK;
  int j = 0;
  for (; j + 1 < n_full; j += 2) {
    dma_iter<DK, DV, NW, BN, 0, true>(j, n_kt, n_w, tile, vtile, K, V, Ks, Vs, n_s, w, wave_first, st, pf, c, row, h,
                                 Mts, zs, Zs);
    dma_iter<DK, DV, NW, BN, 1, true>(j + 1, n_kt, n_w, tile, vtile, K, V, Ks, Vs, n_s, w, wave_first, st, pf, c, row,
                                 h, Mts, zs, Zs);
  }
  for (; j < n_kt; j += 2) {  // j is even here
    dma_iter<DK, DV, NW, BN, 0, false>(j, n_kt, n_w, tile, vtile, K, V, Ks, Vs, n_s, w, wave_first, st, pf, c, row,
                                  h, Mts, zs, Zs);
    if (j + 1 < n_kt)
      dma_iter<DK, DV, NW, BN, 1, false>(j + 1, n_kt, n_w, tile, vtile, K, V, Ks, Vs, n_s, w, wave_first, st, pf, c,
                                    row, h, Mts, zs, Zs);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's part of M^T and z has landed
  __syncthreads();
  if (!wave_on) return;

  // the gate and the output rows, formed after the key loop so that they
  // hold no registers through it
  const float g = 1.f / (1.f + __expf(-a.beta[hq]));
  bf16* O = static_cast<bf16*>(a.out) + (qh * a.L + seg_start) * DV;
  // M^T sits in the buffers the last tile (parity (n_kt - 1) % 2) freed
  const bool pl = ((n_kt - 1) & 1) != 0;
  const bf16* Ma = pl ? Ks[1] : Ks[0];
  const bf16* Mb = pl ? Vs[0] : Vs[1];
  float l = st.l0 + st.l1;
  l = xhalf_sum(l);
  if (a.lse != nullptr && h == 0 && row < n_s)
    a.lse[qh * a.L + seg_start + row] = st.m_run * c + __log2f(l);
  float sq[NC][8];
  float dp = 0.f;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = feature_map((float)st.qf[cc][e]);
      sq[cc][e] = s;
      dp += s * Zs[16 * cc + 8 * h + e];
    }
  const float den = xhalf_sum(dp);
  const float ca = (1.f - g) / l, cm = g / den;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[db][r] *= ca;
  bf16x8 sf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) sf[cc][e] = (bf16)(sq[cc][e] * cm);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      mma32(st.oacc[db],
            load8<bf16>(lds_at(db >= 2 ? Mb : Ma, (st.ko ^ (32u * cc)) + 2 * 32 * (db & 1) * DK)),
            sf[cc]);
  if (row < n_s) {
    bf16* orow = O + (int64_t)row * DV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = (bf16)st.oacc[db][4 * rq + j];
        store4<bf16>(orow + 32 * db + 8 * rq + 4 * h, y);
      }
  }
}

template <typename T, int D, int NW>
hipError_t launch_attn_t(const AttnArgs& a, int64_t units, hipStream_t stream) {
  constexpr int BN = 64;
  const int64_t G = a.Hq / a.Hkv;
  const int64_t total = units * a.s_count * a.n_qt * G;
  if constexpr (sizeof(T) == 2 && (D == 64 || D == 128)) {
    bool packed = false;
    if constexpr (NW == 4) {
      if (G % NW == 0) {
        packed = true;
        hipLaunchKernelGGL((attn_kernel_dma<D, D, NW, BN, true>), dim3((unsigned)total),
                           dim3(NW * 64), 0, stream, a);
      }
    }
    if (!packed)
      hipLaunchKernelGGL((attn_kernel_dma<D, D, NW, BN, false>), dim3((unsigned)total),
                         dim3(NW * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<T, D, D, NW, BN>), dim3((unsigned)total), dim3(NW * 64), 0,
                       stream, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attn_w(const AttnArgs& a, int64_t units, hipStream_t stream) {
  switch (attn_waves(a.seg_len < a.L ? a.seg_len : a.L)) {
    case 1: return launch_attn_t<T, D, 1>(a, units, stream);
    case 2: return launch_attn_t<T, D, 2>(a, units, stream);
    default: return launch_attn_t<T, D, 4>(a, units, stream);
  }
}

template <typename T>
hipError_t launch_attn_d(int d, const AttnArgs& a, int64_t units, hipStream_t stream) {
  switch (d) {
    case 32: return launch_attn_w<T, 32>(a, units, stream);
    case 64: return launch_attn_w<T, 64>(a, units, stream);
    case 128: return launch_attn_w<T, 128>(a, units, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int attn_waves(int64_t seg_len) { return seg_len <= 32 ? 1 : (seg_len <= 64 ? 2 : 4); }

hipError_t launch_attn(int dtype, int d, const AttnArgs& a, int64_t units, hipStream_t stream) {
  return dtype == kBF16 ? launch_attn_d<bf16>(d, a, units, stream)
                        : launch_attn_d<float>(d, a, units, stream);
}

namespace {

// d_key != d_value, four waves (rows past a short segment's end are masked),
// every ordered pair of distinct widths in {32, 64, 128}: bf16 with both
// widths in {64, 128} on the DMA kernel, the rest on the register-staged one.
template <typename T, int DK, int DV>
hipError_t launch_attn_kv_t(const AttnArgs& a, int64_t units, hipStream_t stream) {
  constexpr int NW = 4, BN = 64;
  const int64_t G = a.Hq / a.Hkv;
  const int64_t total = units * a.s_count * a.n_qt * G;
  if constexpr (sizeof(T) == 2 && (DK == 64 || DK == 128) && (DV == 64 || DV == 128)) {
    if (G % NW == 0)
      hipLaunchKernelGGL((attn_kernel_dma<DK, DV, NW, BN, true>), dim3((unsigned)total),
                         dim3(NW * 64), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_kernel_dma<DK, DV, NW, BN, false>), dim3((unsigned)total),
                         dim3(NW * 64), 0, stream, a);
  } else
    hipLaunchKernelGGL((attn_kernel<T, DK, DV, NW, BN>), dim3((unsigned)total), dim3(NW * 64),
                       0, stream, a);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_attn_kv_v(int dv, const AttnArgs& a, int64_t units, hipStream_t stream) {
  switch (dv) {
    case 32: return DK != 32 ? launch_attn_kv_t<T, DK, 32>(a, units, stream) : hipErrorInvalidValue;
    case 64: return DK != 64 ? launch_attn_kv_t<T, DK, 64>(a, units, stream) : hipErrorInvalidValue;
    case 128: return DK != 128 ? launch_attn_kv_t<T, DK, 128>(a, units, stream) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_attn_kv_d(int dk, int dv, const AttnArgs& a, int64_t units, hipStream_t stream) {
  switch (dk) {
    case 32: return launch_attn_kv_v<T, 32>(dv, a, units, stream);
    case 64: return launch_attn_kv_v<T, 64>(dv, a, units, stream);
    case 128: return launch_attn_kv_v<T, 128>(dv, a, units, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_kv(int dtype, int dk, int dv, const AttnArgs& a, int64_t units,
                          hipStream_t stream) {
  return dtype == kBF16 ? launch_attn_kv_d<bf16>(dk, dv, a, units, stream)
                        : launch_attn_kv_d<float>(dk, dv, a, units, stream);
}

}  // namespace infini
