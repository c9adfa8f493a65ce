// Gradients of the local causal attention, bf16 with MFMA (d in {64, 128}).
//
// "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
// block?" (A_dot) and "How is an Infini-attention model trained?". With the
// forward's softmax statistics lse (base-2, scaled scores), P_tu =
// exp2(c q_t . k_u - lse_t), c = log2(e) / sqrt(d); dA_dot = (1 - g) dout;
// dS_tu = P_tu ((1 - g) dout_t . v_u - delta_t):
//   dQ_t = sum_u dS_tu k_u / sqrt(d)            (query-major kernel)
//   dK_u = sum_t dS_tu q_t / sqrt(d), dV_u = sum_t P_tu (1 - g) dout_t
//                                              (key-major kernel, over the
//                                               query heads of the group)
// Tiles come into LDS by DMA in the row-major "K" layout (lds_tile.hpp); a
// tile is read row-wise for one operand and with transposing reads for the
// other, so each tensor is staged once.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace infini {

namespace {

constexpr int kNW = 4;     // waves per workgroup
constexpr int kMaxG = 64;  // query heads per KV head in the key-major kernel

// Round-robin rows (query or key) over the waves: row index base + w + 4 i
// for lane i, so every wave meets the causal diagonal in the same tiles.

// ---- dQ: one workgroup per 128 query rows, key tiles of 64 ---------------------

template <int D>
struct DqLane {
  static constexpr int NC = D / 16, NDB = D / 32;
  bf16x8 qf[NC], dof[NC];  // B operands: query row, k = head dim
  f32x16 acc[NDB];         // dQ^T
  uint32_t ko;             // row read offset (as the forward's K reads)
  uint32_t tk[2][NDB];     // transposing read offsets of K
};

// One 64-key tile: S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
// MASK: the tile reaches the causal diagonal. Key k0 + 32 kb + acc_row(r, h)
// lies after the lane's row where 32 kb + 8 (r / 4) + r % 4 exceeds the
// lane's threshold kt = row - 4 h - k0.
template <int D, bool MASK>
__device__ __forceinline__ void dq_tile(const bf16* Kt, const bf16* Vt, DqLane<D>& st, float c,
                                        float lse, float dl, float om, int kt) {
  constexpr int NC = D / 16, NDB = D / 32;
  f32x16 sacc[2], pacc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    sacc[kb] = zero16();
    pacc[kb] = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const uint32_t o = (st.ko ^ (32u * cc)) + 2 * 32 * kb * D;
      mma32(sacc[kb], load8<bf16>(lds_at(Kt, o)), st.qf[cc]);
      mma32(pacc[kb], load8<bf16>(lds_at(Vt, o)), st.dof[cc]);
    }
  }
  bf16x8 dsf[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c, -lse));
      if (MASK && 32 * kb + 8 * (r >> 2) + (r & 3) > kt) p = 0.f;
      dsf[2 * kb + (r >> 3)][r & 7] = (bf16)(p * __builtin_fmaf(om, pacc[kb][r], -dl));
    }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int pc = 0; pc < 4; ++pc)
      mma32(st.acc[db], tr_frag_k<D>(Kt, st.tk[0][db], st.tk[1][db], pc), dsf[pc]);
}

template <int D>
__global__ __launch_bounds__(kNW * 64, 2) void dq_kernel(BwdArgs a, int n_qt) {
  constexpr int BN = 64, BM = 32 * kNW, NC = D / 16, NDB = D / 32;
  __shared__ __align__(1024) bf16 Ks0[BN * D];
  __shared__ __align__(1024) bf16 Ks1[BN * D];
  __shared__ __align__(1024) bf16 Vs0[BN * D];
  __shared__ __align__(1024) bf16 Vs1[BN * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  // XCD-aware order as in the forward: a contiguous range of logical tiles
  // per XCD, heaviest query tiles of a (unit, segment) group first
  int t = blockIdx.x;
  {
    const int per = (int)(gridDim.x >> 3);
    if (t < per * 8) t = (t & 7) * per + (t >> 3);
  }
  const int G = a.Hq / a.Hkv;
  const int in_grp = n_qt * G;
  const int grp = t / in_grp, rr = t % in_grp;
  const int qt = n_qt - 1 - rr / G, hg = rr % G;
  const int sl = grp % a.S, unit = grp / a.S;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv, hq = kvh * G + hg;
  const int64_t seg_start = (int64_t)sl * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  const int q0 = qt * BM;
  if (q0 >= n_s) return;

  const int64_t qh = (int64_t)b * a.Hq + hq;
  const int64_t rbase = qh * a.L + seg_start;  // row index of the segment's first query
  const bf16* K = static_cast<const bf16*>(a.k) + ((int64_t)unit * a.L + seg_start) * D;
  const bf16* V = static_cast<const bf16*>(a.v) + ((int64_t)unit * a.L + seg_start) * D;
  const float om = 1.f - 1.f / (1.f + __expf(-a.beta[hq]));
  const float c = a.scale_log2;
  const int row = q0 + w + kNW * i;
  const bool live = row < n_s;
  const int n_kt = (min(q0 + BM, n_s) + BN - 1) / BN;

  DmaTile<D, kNW, BN> tile;
  tile.init(w, lane);
  tile.template issue<true>(K, Ks0, 0, n_s, w);
  tile.template issue<true>(V, Vs0, 0, n_s, w);

  DqLane<D> st;
  st.ko = 2 * (i * D + 8 * (h ^ swz_k<D>(i)));
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    st.tk[0][db] = tr_offset_k<D>(lane, db, 0);
    st.tk[1][db] = tr_offset_k<D>(lane, db, 1);
    st.acc[db] = zero16();
  }
  const bf16* Q = static_cast<const bf16*>(a.q) + (rbase + row) * D;
  const bf16* dO = static_cast<const bf16*>(a.dout) + (rbase + row) * D;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    st.qf[cc] = live ? load8<bf16>(Q + 16 * cc + 8 * h) : zero_frag<bf16>();
    st.dof[cc] = live ? load8<bf16>(dO + 16 * cc + 8 * h) : zero_frag<bf16>();
  }
  // rows past the segment: lse = +inf gives P = 0
  const float lse = live ? a.lse[rbase + row] : INFINITY;
  const float dl = live ? a.delta[rbase + row] : 0.f;
  const int kt0 = row - 4 * h;  // the causal threshold of key tile k0 is kt0 - k0
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  bf16* const Ks[2] = {Ks0, Ks1};
  bf16* const Vs[2] = {Vs0, Vs1};
  // Tile j on buffer parity P = j % 2 (a constant). Every tile loads its
  // successor (the last one reloads itself, in bounds and unused) into the
  // other buffers first and waits for it at its end: with the load and the
  // wait unconditional, the compiler sees that a tile's reads touch only
  // buffers no load is filling, and does not wait for the load.
  auto step = [&](int j, auto par, auto mask) {
    constexpr int P = decltype(par)::value;
    const int jn = min(j + 1, n_kt - 1);
    tile.template issue<true>(K, Ks[P ^ 1], jn * BN, n_s, w);
    tile.template issue<true>(V, Vs[P ^ 1], jn * BN, n_s, w);
    const int k0 = j * BN;
    dq_tile<D, decltype(mask)::value>(Ks[P], Vs[P], st, c, lse, dl, om, kt0 - k0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Key tiles that end before the block's first query row (k0 + BN <= q0)
  // lie below every row's diagonal and take no mask. Their count q0 / BN is
  // even (q0 is a multiple of 2 BN) and below n_kt, so the masked tiles
  // start on buffer parity 0.
  static_assert(BM % (2 * BN) == 0, "even count of unmasked key tiles");
  const int n_free = q0 / BN;
  for (int j = 0; j < n_free; j += 2) {
    step(j, std::integral_constant<int, 0>{}, std::false_type{});
    step(j + 1, std::integral_constant<int, 1>{}, std::false_type{});
  }
  for (int j = n_free; j < n_kt; j += 2) {
    step(j, std::integral_constant<int, 0>{}, std::true_type{});
    if (j + 1 < n_kt) step(j + 1, std::integral_constant<int, 1>{}, std::true_type{});
  }
  // The retrieval part of dQ, (M dn^T + dden z) sigma'(q): the snapshot M^T
  // comes into the K buffers (free after the last tile), dn (bf16, written
  // by the retrieval kernel) is read straight into the B operand in the
  // accumulator-derived order tr_frag_k expects (fragment pc of 64-row tile
  // ts holds columns 64 ts + 16 pc + 4 h + 0..3 and + 8 .. + 11).
  constexpr int NT = D / 64;
  const bf16* Mt = static_cast<const bf16*>(a.snapM) + ((int64_t)unit * a.S + sl) * D * D;
  tile.template issue<true>(Mt, Ks0, 0, D, w);
  if constexpr (NT > 1) tile.template issue<true>(Mt, Ks1, 64, D, w);
  const bf16* dnr = static_cast<const bf16*>(a.dn) + (rbase + row) * D;
  bf16x8 dnf[NT][4];
#pragma unroll
  for (int ts = 0; ts < NT; ++ts)
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) {
      const int j0 = 64 * ts + 16 * pc + 4 * h;
      dnf[ts][pc] = live ? load4x2<bf16>(dnr + j0, dnr + j0 + 8) : zero_frag<bf16>();
    }
  const float dden = live ? a.dden[rbase + row] : 0.f;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 racc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    racc[db] = zero16();
#pragma unroll
    for (int ts = 0; ts < NT; ++ts)
#pragma unroll
      for (int pc = 0; pc < 4; ++pc)
        mma32(racc[db], tr_frag_k<D>(Ks[ts], st.tk[0][db], st.tk[1][db], pc), dnf[ts][pc]);
  }
  if (!live) return;
  // dq = dQ^T^T / sqrt(d) + (dQ_ret + dden z) sigma'(q)
  const float inv_sqrt_d = a.scale_log2 / kLog2e;
  const float* z = a.snapZ + ((int64_t)unit * a.S + sl) * D;
  bf16* dq = static_cast<bf16*>(a.dq) + (rbase + row) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int col = 32 * db + 8 * rq + 4 * h;
      const bf16x4 q4 = load4<bf16>(Q + col);
      const f32x4 z4 = *reinterpret_cast<const f32x4*>(z + col);
      bf16x4 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = (float)q4[j];
        const float ds = x > 0.f ? 1.f : __builtin_amdgcn_exp2f(x * kLog2e);
        y[j] = (bf16)(st.acc[db][4 * rq + j] * inv_sqrt_d +
                      (racc[db][4 * rq + j] + dden * z4[j]) * ds);
      }
      store4<bf16>(dq + col, y);
    }
}

// ---- dK, dV: one workgroup per 128 keys, query tiles of 32, all G heads -------

// A tile load as DmaTile::issue<true>, but with rows past the segment's end
// read as zeros: the resource covers only the valid rows and the buffer's
// range check zero-fills the rest. The whole offset goes in the lane's
// register, since the range check leaves out the scalar offset.
template <int D, int NW, int BN>
__device__ __forceinline__ void issue_zero_tail(const DmaTile<D, NW, BN>& t, const bf16* X,
                                                bf16* Xs, int k0, int n_s, int w) {
  using Tile = DmaTile<D, NW, BN>;
  const int rows = min(BN, n_s - k0);
  const __amdgpu_buffer_rsrc_t rx = raw_rsrc(X + (int64_t)k0 * D, (uint32_t)rows * D * 2);
#pragma unroll
  for (int j = 0; j < Tile::PER_WAVE; ++j) {
    const int blk = (j * NW + w) * 64 * 8;
    const uint32_t xj = Tile::J_INV ? t.k_off[0] + j * Tile::J_STEP : t.k_off[j];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(Xs + blk), 16, xj, 0, 0, 0);
  }
}

template <int D>
struct KvLane {
  static constexpr int NC = D / 16, NDB = D / 32;
  bf16x8 kf[NC];            // B operand: key row, k = head dim (V's is read from LDS)
  f32x16 dk[NDB], dv[NDB];  // dK^T, dV^T
  uint32_t ko;              // row read offset in a query tile
  uint32_t vo;              // row read offset of this lane's key in the V block
  uint32_t tk[2][NDB];
};

// One 32-query tile of one head: S = Q K^T, dP = dO V^T, P, dS;
// dV^T += dO^T P, dK^T += Q^T dS. Rows past the segment's end come in as
// zeros (Q, dO, lse, delta): P = 1 there but dP = dS = 0 and dO = 0, so they
// add nothing and need no mask. The causal mask drops P where key > q, i.e.
// where this lane's threshold kq = key - q0 - 4 h exceeds the row's offset
// 8 g4 + j in the tile; MASK: the tile reaches the diagonal (off it every
// row follows every key of the block and the mask is left out).
template <int D, bool MASK>
__device__ __forceinline__ void kv_tile(const bf16* Qt, const bf16* Ot, const bf16* Vb,
                                        const float* lse_t, const float* dl_t, KvLane<D>& st,
                                        float c, float om, int h, int kq) {
  constexpr int NC = D / 16, NDB = D / 32;
  f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const uint32_t o = st.ko ^ (32u * cc);
    mma32(sacc, load8<bf16>(lds_at(Qt, o)), st.kf[cc]);
    mma32(pacc, load8<bf16>(lds_at(Ot, o)), load8<bf16>(lds_at(Vb, st.vo ^ (32u * cc))));
  }
  bf16x8 pf[2], dsf[2];
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    // rows 8 g4 + 4 h + 0..3 of the tile
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_t + 8 * g4 + 4 * h);
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(dl_t + 8 * g4 + 4 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * g4 + j;
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -l4[j]));
      if (MASK && kq > 8 * g4 + j) p = 0.f;
      pf[r >> 3][r & 7] = (bf16)(p * om);
      dsf[r >> 3][r & 7] = (bf16)(p * __builtin_fmaf(om, pacc[r], -d4[j]));
    }
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int pc = 0; pc < 2; ++pc) {
      mma32(st.dv[db], tr_frag_k<D>(Ot, st.tk[0][db], st.tk[1][db], pc), pf[pc]);
      mma32(st.dk[db], tr_frag_k<D>(Qt, st.tk[0][db], st.tk[1][db], pc), dsf[pc]);
    }
}

template <int D>
__global__ __launch_bounds__(kNW * 64, 2) void kv_kernel(BwdArgs a, int n_kt) {
  constexpr int BQ = 32, BK = 32 * kNW, NC = D / 16, NDB = D / 32;
  __shared__ __align__(1024) bf16 Qs0[BQ * D];
  __shared__ __align__(1024) bf16 Qs1[BQ * D];
  __shared__ __align__(1024) bf16 Os0[BQ * D];
  __shared__ __align__(1024) bf16 Os1[BQ * D];
  __shared__ __align__(1024) bf16 Vb[BK * D];  // V of the workgroup's keys
  __shared__ __align__(16) float Ls0[64], Ls1[64], Ds0[64], Ds1[64];
  __shared__ float omg[kMaxG];  // 1 - sigmoid(beta) of the group's query heads

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  int t = blockIdx.x;
  {
    const int per = (int)(gridDim.x >> 3);
    if (t < per * 8) t = (t & 7) * per + (t >> 3);
  }
  const int kt = t % n_kt, grp = t / n_kt;  // key tiles of a segment: heaviest first
  const int sl = grp % a.S, unit = grp / a.S;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int64_t seg_start = (int64_t)sl * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  const int k0 = kt * BK;
  if (k0 >= n_s) return;
  const int key = k0 + w + kNW * i;
  const bool live = key < n_s;
  const float c = a.scale_log2;

  KvLane<D> st;
  const int64_t krow = (int64_t)unit * a.L + seg_start + key;
  {  // The V rows of the block, by DMA (rows past the segment repeat its
     // last). LDS row 32 w' + i' holds key w' + NW i', so that the 16 lanes
     // of a read (one wave, consecutive i) take 16 consecutive rows: with the
     // K swizzle, no bank conflicts (key order would put them 4 rows apart).
    constexpr int CPR = D / 8, PER = BK * CPR / 64 / kNW;
    const int rows = min(BK, n_s - k0);
    const __amdgpu_buffer_rsrc_t rv = raw_rsrc(
        static_cast<const bf16*>(a.v) + ((int64_t)unit * a.L + seg_start + k0) * D,
        (uint32_t)rows * D * 2);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int p = (j * kNW + w) * 64 + lane;  // physical chunk of the block
      const int R = p / CPR, phys = p % CPR;
      const int r = min((R >> 5) + kNW * (R & 31), rows - 1);
      const uint32_t off = 2 * (r * D + 8 * (phys ^ swz_k<D>(R)));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(Vb + (j * kNW + w) * 64 * 8), 16,
                                               off, 0, 0, 0);
    }
  }
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
    st.kf[cc] = live ? load8<bf16>(static_cast<const bf16*>(a.k) + krow * D + 16 * cc + 8 * h)
                     : zero_frag<bf16>();
  st.ko = 2 * (i * D + 8 * (h ^ swz_k<D>(i)));
  {
    const int R = 32 * w + i;  // LDS row of this lane's key (w + NW i)
    st.vo = 2 * (R * D + 8 * (h ^ swz_k<D>(R)));
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    st.tk[0][db] = tr_offset_k<D>(lane, db, 0);
    st.tk[1][db] = tr_offset_k<D>(lane, db, 1);
    st.dk[db] = zero16();
    st.dv[db] = zero16();
  }

  if (tid < G) omg[tid] = 1.f - 1.f / (1.f + __expf(-a.beta[kvh * G + tid]));
  DmaTile<D, kNW, BQ> tile;
  tile.init(w, lane);
  bf16* const Qs[2] = {Qs0, Qs1};
  bf16* const Os[2] = {Os0, Os1};
  auto Ls = [&](int P) { return P ? Ls1 : Ls0; };
  auto Ds = [&](int P) { return P ? Ds1 : Ds0; };
  // query tiles q0 = k0, k0 + 32, ... of every head of the group, as one
  // list of items (head hg, tile qi), head-major. The position is carried as
  // scalar counters: dividing the item index would put hg and qi in vector
  // registers, and every DMA built from them would become a waterfall loop.
  const int n_q = (n_s - k0 + BQ - 1) / BQ;
  // The group's first query head row, made explicitly scalar: the same
  // product also indexes beta under the divergent branch above, and merged
  // through that branch it would reach the DMA descriptors in a vector register.
  const int hrow0 = __builtin_amdgcn_readfirstlane(b * a.Hq + kvh * G);
  auto issue = [&](int hg, int qi, bf16* Qd, bf16* Od, float* Ld, float* Dd) {
    const int q0 = k0 + qi * BQ;
    const int64_t rb = (int64_t)(hrow0 + hg) * a.L + seg_start;
    issue_zero_tail(tile, static_cast<const bf16*>(a.q) + rb * D, Qd, q0, n_s, w);
    issue_zero_tail(tile, static_cast<const bf16*>(a.dout) + rb * D, Od, q0, n_s, w);
    // 32 floats of lse (wave 0) and delta (wave 1); lanes past the rows read zeros
    const int bytes = min(BQ, n_s - q0) * 4;
    if (w == 0) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(a.lse + rb + q0), 0, bytes, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)Ld, 4, lane * 4, 0, 0, 0);
    } else if (w == 1) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          a.delta + rb + q0, 0, bytes, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)Dd, 4, lane * 4, 0, 0, 0);
    }
  };
  issue(0, 0, Qs0, Os0, Ls0, Ds0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int kq0 = key - 4 * h - k0;  // the causal threshold of tile qi is kq0 - BQ qi
  // Item order: the tiles that reach the diagonal (qi < n_d) of every head,
  // then the interior tiles of every head, each part head-major; the second
  // part takes no mask.
  const int n_d = min(BK / BQ, n_q);
  auto succ = [&](int& hn, int& qn) {  // (hn, qn) <- its successor; the last item keeps itself
    const bool d = qn < n_d;
    if (qn + 1 < (d ? n_d : n_q)) {
      ++qn;
    } else if (hn + 1 < G) {
      ++hn;
      qn = d ? 0 : n_d;
    } else if (d && n_d < n_q) {
      hn = 0;
      qn = n_d;
    }
  };
  int hg = 0, qi = 0;
  // as in dq_kernel: every item loads its successor (the last reloads
  // itself) and waits for it, unconditionally
  auto step = [&](auto par, auto mask) {
    constexpr int P = decltype(par)::value;
    int hn = hg, qn = qi;
    succ(hn, qn);
    issue(hn, qn, Qs[P ^ 1], Os[P ^ 1], Ls(P ^ 1), Ds(P ^ 1));
    kv_tile<D, decltype(mask)::value>(Qs[P], Os[P], Vb, Ls(P), Ds(P), st, c, omg[hg], h,
                                      kq0 - BQ * qi);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    hg = hn;
    qi = qn;
  };
  // There are interior tiles only when n_d = BK / BQ, an even number, so the
  // first part's item count is then even and the second starts on parity 0.
  static_assert((BK / BQ) % 2 == 0, "even count of diagonal items");
  const int n1 = G * n_d, n2 = G * (n_q - n_d);
  for (int it = 0; it < n1; it += 2) {
    step(std::integral_constant<int, 0>{}, std::true_type{});
    if (it + 1 < n1) step(std::integral_constant<int, 1>{}, std::true_type{});
  }
  for (int it = 0; it < n2; it += 2) {
    step(std::integral_constant<int, 0>{}, std::false_type{});
    if (it + 1 < n2) step(std::integral_constant<int, 1>{}, std::false_type{});
  }
  if (!live) return;
  const float inv_sqrt_d = a.scale_log2 / kLog2e;
  float* dk = a.dk_acc + krow * D;
  float* dv = a.dv_acc + krow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int col = 32 * db + 8 * rq + 4 * h;
      f32x4 yk, yv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        yk[j] = st.dk[db][4 * rq + j] * inv_sqrt_d;
        yv[j] = st.dv[db][4 * rq + j];
      }
      *reinterpret_cast<f32x4*>(dk + col) = yk;
      *reinterpret_cast<f32x4*>(dv + col) = yv;
    }
}

// ---- retrieval, fused: one workgroup per 128 query rows of one head ---------
//
// "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
// block?": A_mem = sigma(q) M / (sigma(q) . z) with M = M_{s-1}, z = z_{s-1},
// out = g A_mem + (1 - g) A_dot. For each query row t, from d_out, out and
// the forward's snapshot (M^T in bf16, z in float):
//   n = sigma(q) M, den = sigma(q) . z, A_mem = n / den,
//   dam = d_out . A_mem, doo = d_out . out,
//   delta_t = doo - g dam (the softmax row term: out - g A_mem = (1 - g) A_dot),
//   dg_t = (dam - doo) / (1 - g), dden_t = -g dam / den, dn = g d_out / den,
// and dn itself (bf16). The query-major kernel then adds the retrieval part
// of dQ, (dn M^T + dden_t z) * sigma'(q), in its epilogue; dn also feeds the
// products into dL/dM_{s-1}. n^T = M^T sigma(q)^T runs on the matrix cores
// with M^T in LDS (the K layout), as the query-major kernel forms S^T.
// sigma(q) enters the product in bf16, den in float. Three waves per SIMD:
// at d = 128 that leaves 168 registers, and a few row indices of the final
// stores go to scratch, which costs less than the third wave gains.
template <int D>
__global__ __launch_bounds__(kNW * 64, 3) void retr_kernel(BwdArgs a, int n_qt) {
  constexpr int BM = 32 * kNW, NC = D / 16, NT = D / 64, NJB = D / 32;
  __shared__ __align__(1024) bf16 Ms0[64 * D];
  __shared__ __align__(1024) bf16 Ms1[NT > 1 ? 64 * D : 8];
  __shared__ __align__(16) float zs[D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  // the query-major kernel's tile order: the query tiles and heads of one
  // (unit, segment), which share its snapshot, run together on one XCD
  int t = blockIdx.x;
  {
    const int per = (int)(gridDim.x >> 3);
    if (t < per * 8) t = (t & 7) * per + (t >> 3);
  }
  const int G = a.Hq / a.Hkv;
  const int in_grp = n_qt * G;
  const int grp = t / in_grp, rr = t % in_grp;
  const int qt = rr / G, hg = rr % G;
  const int sl = grp % a.S, unit = grp / a.S;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv, hq = kvh * G + hg;
  const int64_t seg_start = (int64_t)sl * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  const int q0 = qt * BM;
  if (q0 >= n_s) return;
  const int64_t rbase = ((int64_t)b * a.Hq + hq) * a.L + seg_start;
  const int row = q0 + w + kNW * i;
  const bool live = row < n_s;

  const bf16* Mt = static_cast<const bf16*>(a.snapM) + ((int64_t)unit * a.S + sl) * D * D;
  DmaTile<D, kNW, 64> tile;
  tile.init(w, lane);
  tile.template issue<true>(Mt, Ms0, 0, D, w);
  if constexpr (NT > 1) tile.template issue<true>(Mt, Ms1, 64, D, w);
  if (tid < D) zs[tid] = a.snapZ[((int64_t)unit * a.S + sl) * D + tid];

  const bf16* Q = static_cast<const bf16*>(a.q) + (rbase + row) * D;
  const bf16* O = static_cast<const bf16*>(a.out) + (rbase + row) * D;
  const bf16* dO = static_cast<const bf16*>(a.dout) + (rbase + row) * D;
  bf16x8 qf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) qf[cc] = live ? load8<bf16>(Q + 16 * cc + 8 * h) : zero_frag<bf16>();
  const float g = 1.f / (1.f + __expf(-a.beta[hq]));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // sigma(q): bf16 operand of n^T, float in den (this lane's half of the columns)
  bf16x8 sqf[NC];
  float den = 0.f;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sg = feature_map((float)qf[cc][e]);
      sqf[cc][e] = (bf16)sg;
      den += sg * zs[16 * cc + 8 * h + e];
    }
  den = xhalf_sum(den);

  // n^T = M^T sigma(q)^T with the rows of each 32-row block of M^T read in
  // the order pi(i) = i ^ 12 where bits 2 and 3 of i differ (row groups
  // 4..7 <-> 8..11, 20..23 <-> 24..27): accumulator register 8 m + e of lane
  // (i, h) then holds column 32 jb + 16 m + 8 h + e of n, the columns of the
  // lane's 16-byte d_out chunks below. pi keeps each 16-row half's set of
  // rows, so the swizzle's reads stay free of bank conflicts.
  __builtin_amdgcn_sched_barrier(0);  // sigma(q) complete before the product
  bf16* const Ms[2] = {Ms0, NT > 1 ? Ms1 : Ms0};
  const int pi = i ^ ((((i >> 2) ^ (i >> 3)) & 1) * 12);
  const uint32_t ko = 2 * (pi * D + 8 * (h ^ swz_k<D>(pi)));
  f32x16 nacc[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    nacc[jb] = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const uint32_t o = (ko ^ (32u * cc)) + 2 * 32 * (jb & 1) * D;
      mma32(nacc[jb], load8<bf16>(lds_at(Ms[jb >> 1], o)), sqf[cc]);
    }
  }

  // d_out and out come in 16-byte chunks: lane (i, h) loads columns
  // 32 jb + 16 m + 8 h + 0..7 of row `row` (32 contiguous bytes of the row
  // per lane pair and instruction), the columns of its n accumulators 8 m ..
  // 8 m + 7. dn = g d_out / den is stored (bf16) for the query-major kernel,
  // which forms the retrieval part of dQ from it, and for the products into
  // dL/dM_{s-1}.
  const float inv_den = 1.f / den;
  const float gd = g * inv_den;
  bf16* dn = static_cast<bf16*>(a.dn) + (rbase + row) * D;
  // The segment's first row (row 0) attends to its own key alone, so A_dot
  // is v_0 and out = g A_mem + (1 - g) v_0: that row reads v_0 in place of
  // its output row and forms delta = (1 - g) d_out . v_0 and d(gate) =
  // d_out . A_mem - d_out . v_0 exactly. From the stored output, whose
  // rounding would not cancel against (1 - g) d_out . v_0 in dS (exactly
  // zero there), the rounding would land whole in that row's dQ.
  const bf16* Or = row == 0 ? static_cast<const bf16*>(a.v) + ((int64_t)unit * a.L + seg_start) * D
                            : O;
  // every load before the first store (the stores could alias them as far
  // as the compiler knows, so it would not move a load above one)
  bf16x8 d8[NJB][2], o8[NJB][2];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int col = 32 * jb + 16 * m + 8 * h;
      d8[jb][m] = live ? load8<bf16>(dO + col) : zero_frag<bf16>();
      o8[jb][m] = live ? load8<bf16>(Or + col) : zero_frag<bf16>();
    }
  float dam = 0.f, doo = 0.f;
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dv = (float)d8[jb][m][e];
        dam += dv * nacc[jb][8 * m + e];
        doo += dv * (float)o8[jb][m][e];
        y[e] = (bf16)(gd * dv);
      }
      if (live) store8<bf16>(dn + 32 * jb + 16 * m + 8 * h, y);
    }
  dam = xhalf_sum(dam);
  doo = xhalf_sum(doo);
  dam *= inv_den;
  const float dden = -g * dam * inv_den;
  if (live && h == 0) {
    // row 0 (doo = d_out . v_0): out = g A_mem + (1 - g) v_0 exactly
    a.delta[rbase + row] = row == 0 ? (1.f - g) * doo : doo - g * dam;
    a.dg[rbase + row] = row == 0 ? dam - doo : (dam - doo) / (1.f - g);
    a.dden[rbase + row] = dden;
  }
}

// ---- the memory update's backward, fused: one workgroup per 128 key rows ----
//
// "Infini-Attention" (AI Wiki), "How does the compressive memory work?": with
// Phi = sigma(K_s), c_t = Phi_t . z_{s-1},
//   linear: M_s = M_{s-1} + Phi^T V
//   delta:  M_s = M_{s-1} + Phi^T R, R = V - P / c, P = Phi M_{s-1}.
// Given dM_s (the reversed chain's snapshot, dM_s^T in bf16), per key row t:
//   du_t = Phi_t dM_s                  (dL/dR_t, or dL/dV_t for the linear rule)
//   dv_t = dv_acc_t + du_t             (the output itself)
//   delta: dP_t = -du_t / c_t, dc_t = (du_t . P_t / c_t) / c_t,
//          dphi_t = R_t dM_s^T + dP_t M_{s-1}^T
//   linear: dphi_t = V_t dM_s^T
// (dz_s, dc_t z and sigma' are added when dK is assembled). U^T = dM_s^T Phi^T
// and P^T = M_{s-1}^T Phi^T take row reads of the snapshots (K layout, in
// LDS) with Phi in the B operand, as the retrieval kernel forms n^T; dphi^T =
// dM_s R^T + M_{s-1} dP^T takes transposing reads, with R and dP in the
// accumulator-derived fragment order tr_frag_k expects. R and dP enter the
// products in bf16, c and everything per element in float.
template <int D, bool DELTA>
__global__ __launch_bounds__(kNW * 64, 2) void upd_kernel(BwdArgs a, int n_kt) {
  constexpr int BK = 32 * kNW, NC = D / 16, NT = D / 64, NJB = D / 32;
  __shared__ __align__(1024) bf16 Us0[64 * D];  // dM_s^T
  __shared__ __align__(1024) bf16 Us1[NT > 1 ? 64 * D : 8];
  __shared__ __align__(1024) bf16 Ps0[DELTA ? 64 * D : 8];  // M_{s-1}^T
  __shared__ __align__(1024) bf16 Ps1[DELTA && NT > 1 ? 64 * D : 8];
  __shared__ __align__(16) float zs[D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  int t = blockIdx.x;
  {
    const int per = (int)(gridDim.x >> 3);
    if (t < per * 8) t = (t & 7) * per + (t >> 3);
  }
  const int kt = t % n_kt, grp = t / n_kt;
  const int sl = grp % a.S, unit = grp / a.S;
  const int64_t seg_start = (int64_t)sl * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  const int k0 = kt * BK;
  if (k0 >= n_s) return;
  const int key = k0 + w + kNW * i;
  const bool live = key < n_s;
  const int64_t row = (int64_t)unit * a.L + seg_start + key;  // [B*Hkv][L] row index
  const int64_t snap = (int64_t)unit * a.S + sl;

  DmaTile<D, kNW, 64> tile;
  tile.init(w, lane);
  const bf16* dMt = static_cast<const bf16*>(a.dMsnap) + snap * D * D;
  tile.template issue<true>(dMt, Us0, 0, D, w);
  if constexpr (NT > 1) tile.template issue<true>(dMt, Us1, 64, D, w);
  if constexpr (DELTA) {
    const bf16* Mt = static_cast<const bf16*>(a.snapM) + snap * D * D;
    tile.template issue<true>(Mt, Ps0, 0, D, w);
    if constexpr (NT > 1) tile.template issue<true>(Mt, Ps1, 64, D, w);
  }
  if (tid < D) zs[tid] = a.snapZ[snap * D + tid];

  const bf16* Kr = static_cast<const bf16*>(a.k) + row * D;
  const bf16* Vr = static_cast<const bf16*>(a.v) + row * D;
  bf16x8 kf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) kf[cc] = live ? load8<bf16>(Kr + 16 * cc + 8 * h) : zero_frag<bf16>();
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Phi: bf16 B operand; c in float (this lane's half of the columns)
  bf16x8 pf[NC];
  float cz = 0.f;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = live ? feature_map((float)kf[cc][e]) : 0.f;
      pf[cc][e] = (bf16)f;
      cz += f * zs[16 * cc + 8 * h + e];
    }
  cz = xhalf_sum(cz);

  bf16* const Us[2] = {Us0, NT > 1 ? Us1 : Us0};
  bf16* const Ps[2] = {Ps0, NT > 1 ? Ps1 : Ps0};
  const uint32_t ko = 2 * (i * D + 8 * (h ^ swz_k<D>(i)));
  f32x16 uacc[NJB], pacc[DELTA ? NJB : 1];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    uacc[jb] = zero16();
    if constexpr (DELTA) pacc[jb] = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const uint32_t o = (ko ^ (32u * cc)) + 2 * 32 * (jb & 1) * D;
      mma32(uacc[jb], load8<bf16>(lds_at(Us[jb >> 1], o)), pf[cc]);
      if constexpr (DELTA) mma32(pacc[jb], load8<bf16>(lds_at(Ps[jb >> 1], o)), pf[cc]);
    }
  }

  // per element: column j = 32 jb + 8 rq + 4 h + 0..3 of row `key`. The
  // update is dv's last term: dv_acc + du goes out as dv itself, rounded once.
  const float ic = 1.f / cz;
  const float* dva = a.dv_acc + row * D;
  bf16* dvo = static_cast<bf16*>(a.dv) + row * D;
  bf16x8 rf[NT][4], df[NT][4];
  float dcs = 0.f;
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int col = 32 * jb + 8 * rq + 4 * h;
      bf16x4 v4;
      f32x4 dv4;
      if (live) {
        v4 = load4<bf16>(Vr + col);
        dv4 = *reinterpret_cast<const f32x4*>(dva + col);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v4[j] = (bf16)0.f;
          dv4[j] = 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * rq + j;
        const float du = uacc[jb][r];
        dv4[j] += du;
        float rv = (float)v4[j], dp = 0.f;
        if constexpr (DELTA) {
          const float pred = pacc[jb][r] * ic;
          rv -= pred;
          dp = -du * ic;
          dcs += du * pred;
        }
        rf[jb >> 1][2 * (jb & 1) + (r >> 3)][r & 7] = (bf16)rv;
        if constexpr (DELTA) df[jb >> 1][2 * (jb & 1) + (r >> 3)][r & 7] = (bf16)dp;
      }
      if (live) {
        bf16x4 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = from_f32<bf16>(dv4[j]);
        store4<bf16>(dvo + col, y);
      }
    }
  if constexpr (DELTA) {
    dcs = xhalf_sum(dcs);
    if (live && h == 0) a.dc[row] = dcs * ic;
  }

  // dphi^T = dM_s R^T (+ M_{s-1} dP^T)
  f32x16 dacc[NJB];
#pragma unroll
  for (int db = 0; db < NJB; ++db) {
    dacc[db] = zero16();
    const uint32_t t0 = tr_offset_k<D>(lane, db, 0), t1 = tr_offset_k<D>(lane, db, 1);
#pragma unroll
    for (int ts = 0; ts < NT; ++ts)
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        mma32(dacc[db], tr_frag_k<D>(Us[ts], t0, t1, pc), rf[ts][pc]);
        if constexpr (DELTA) mma32(dacc[db], tr_frag_k<D>(Ps[ts], t0, t1, pc), df[ts][pc]);
      }
  }
  if (!live) return;
  float* dph = a.dphi + row * D;
#pragma unroll
  for (int db = 0; db < NJB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      f32x4 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = dacc[db][4 * rq + j];
      *reinterpret_cast<f32x4*>(dph + 32 * db + 8 * rq + 4 * h) = y;
    }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.B * a.Hkv;
  const int64_t eff = a.seg_len < a.L ? a.seg_len : a.L;
  const int n_qt = (int)((eff + 32 * kNW - 1) / (32 * kNW));
  const int n_kt = n_qt;  // 128 keys per workgroup
  const int64_t G = a.Hq / a.Hkv;
  const int64_t kv_grid = units * a.S * n_kt, q_grid = units * a.S * n_qt * G;
  if (kv_grid > INT32_MAX || q_grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kv_kernel<D>), dim3((unsigned)kv_grid), dim3(kNW * 64), 0, s, a, n_kt);
  hipLaunchKernelGGL((dq_kernel<D>), dim3((unsigned)q_grid), dim3(kNW * 64), 0, s, a, n_qt);
  return hipGetLastError();
}

template <int D>
hipError_t launch_retr_d(const BwdArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.B * a.Hkv;
  const int64_t eff = a.seg_len < a.L ? a.seg_len : a.L;
  const int n_qt = (int)((eff + 32 * kNW - 1) / (32 * kNW));
  const int64_t grid = units * a.S * n_qt * (a.Hq / a.Hkv);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((retr_kernel<D>), dim3((unsigned)grid), dim3(kNW * 64), 0, s, a, n_qt);
  return hipGetLastError();
}

template <int D>
hipError_t launch_upd_d(const BwdArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.B * a.Hkv;
  const int64_t eff = a.seg_len < a.L ? a.seg_len : a.L;
  const int n_kt = (int)((eff + 32 * kNW - 1) / (32 * kNW));
  const int64_t grid = units * a.S * n_kt;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (a.rule == kRuleDelta)
    hipLaunchKernelGGL((upd_kernel<D, true>), dim3((unsigned)grid), dim3(kNW * 64), 0, s, a, n_kt);
  else
    hipLaunchKernelGGL((upd_kernel<D, false>), dim3((unsigned)grid), dim3(kNW * 64), 0, s, a,
                       n_kt);
  return hipGetLastError();
}

}  // namespace

bool attn_bwd_mfma_supported(int dtype, int d, int group) {
  return dtype == kBF16 && (d == 64 || d == 128) && group <= kMaxG;
}

hipError_t launch_bwd_retrieval_mfma(int d, const BwdArgs& a, hipStream_t stream) {
  switch (d) {
    case 64: return launch_retr_d<64>(a, stream);
    case 128: return launch_retr_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_update_mfma(int d, const BwdArgs& a, hipStream_t stream) {
  switch (d) {
    case 64: return launch_upd_d<64>(a, stream);
    case 128: return launch_upd_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bwd_mfma(int d, const BwdArgs& a, hipStream_t stream) {
  switch (d) {
    case 64: return launch_d<64>(a, stream);
    case 128: return launch_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace infini
