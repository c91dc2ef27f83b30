// Block-sparse attention backward for gfx950: dQ, dK, dV of the forward
// O = softmax(mask(score_mod(Q K^T * scale))) V.
//
// What is computed ("FlexAttention: from rules to fused kernels", section 4: the
// backward recomputes each executed block's scores from the saved row log-sum-exp,
// differentiates score_mod, and walks the same block tables -- a query row's KV list
// for dQ, a KV column's query list for dK and dV, so no atomics are needed):
//   P = exp(score_mod(s) - LSE) on allowed pairs (0 elsewhere), s = (q . k) * scale
//   dV = P^T dO,   dP = dO V^T,   delta_i = sum_d dO_id O_id
//   dS = P * (dP - delta) * d score_mod / d (q . k)
//   dQ = dS K,     dK = dS^T Q
// with d score_mod / d(q . k) = scale (identity, ALiBi, relative position) or
// scale * (1 - tanh^2) (soft-cap).  Gradients are accumulated in fp32 and written
// in fp32; P and dS enter the MFMAs as bf16 (round to nearest even).
//
// gfx950 mapping (16x16 MFMA tiles, wave64; every product on v_mfma_f32_16x16x32_bf16,
// which does twice the work of the 16x16x16 form in the same 16 cycles):
//   * bwd_dkdv_kernel: one workgroup per (b, h_kv, KV block), a wave per 16 keys.  K
//     and V of the wave's keys stay in registers as the B operands of S = Q K^T and
//     dP = dO V^T; the query rows of each listed block (for every query head of the
//     group) are staged in LDS.  dV^T += dO^T P and dK^T += Q^T dS contract over 32
//     query rows at a time: P and dS of two 16-row tiles go straight from the
//     accumulator layout into the B operand, and the A operands are two transposing LDS
//     reads (ds_read_b64_tr_b16) each, in the same row order.
//   * bwd_dq_kernel: one workgroup per (b, h_q, query block), a wave per 16 rows;
//     Q and dO of the wave's rows stay in registers, the K and V tiles of each
//     listed block are staged in LDS, and S^T = K Q^T, dP^T = V dO^T,
//     dQ^T += K^T dS^T (over 32 keys at a time) mirror the first kernel.
//   * bwd_delta_kernel: delta = rowsum(dO * O), D / 8 lanes per row.
// Partial blocks and ragged tails apply the mask rule per element (interpreter).
// The dQ pass also sums the score_mod parameter gradients when asked: ALiBi slopes
// (sum of dS (j - i)) and relative-position table entries (sum of dS per offset), with
// floating-point atomic adds (their order, and so the last bits, may vary per run).
#include "device_common.hpp"
#include "fa_internal.hpp"
#include "prefill_common.hpp"

namespace fa {

namespace {

__device__ __forceinline__ f32x4 mma_k32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 tr_read(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
__device__ __forceinline__ bf16x8 pack8(const float (&x)[8]) {
  const u32x4 v = {cvt_pk_bf16(x[0], x[1]), cvt_pk_bf16(x[2], x[3]), cvt_pk_bf16(x[4], x[5]),
                   cvt_pk_bf16(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, v);
}
// two transposing reads side by side: the A operand of a 16x16x32 product whose
// contraction index k = 8 g + e takes rows base + 4 g + e (e < 4) from the first read and
// rows base + 16 + 4 g + e - 4 from the second
__device__ __forceinline__ bf16x8 cat_tr(const uint8_t* p0, const uint8_t* p1) {
  const u32x2 a = __builtin_bit_cast(u32x2, tr_read(p0));
  const u32x2 b = __builtin_bit_cast(u32x2, tr_read(p1));
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// LDS layout of staged rows.  D = 128: 256-byte rows, 16-byte chunk c of row r stored at
// chunk c ^ (2 (r & 7) + ((r >> 3) & 1)), so the 16 rows that a ds_read_b128 pass reads
// at one chunk land on 16 different chunk positions, and the 8 rows x 32 bytes that a
// pass of transposing reads covers land on all 64 banks once.  D = 64: 144-byte rows
// (128 plus 16 of padding), so a ds_read_b128 pass's 16 rows fall on distinct banks.
template <int D>
struct Lay {
  static constexpr int RS = D == 128 ? 256 : D * 2 + 16;
  // byte offset of bf16 element e (a multiple of 4, below D) of row r
  static __device__ __forceinline__ int off(int r, int e) {
    if constexpr (D == 128) return r * RS + ((((e >> 3) ^ (2 * (r & 7) + ((r >> 3) & 1))) << 4) | ((e & 7) << 1));
    else return r * RS + 2 * e;
  }
};

// Rows [r0, r0 + n) (n <= 128) of a [rows_total, D] bf16 matrix, staged through
// registers: fetch() issues the global loads (zeros past the end) and put() stores them
// to LDS later, so a tile's loads are in flight while the previous tile is computed.
template <int D, int NT>
struct RowStage {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int PER = 128 * CH / NT;        // chunks per thread for 128 rows
  u32x4 r[PER];
  __device__ __forceinline__ void fetch(const uint16_t* src, int r0, int n, int rows_total) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int x = threadIdx.x + u * NT;
      const int row = x / CH, ch = x - row * CH;
      const int gr = r0 + row;
      r[u] = (row < n && gr < rows_total) ? load16(src + (int64_t)gr * D + ch * 8) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void put(uint8_t* dst, int n) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int x = threadIdx.x + u * NT;
      const int row = x / CH, ch = x - row * CH;
      if (row < n) *reinterpret_cast<u32x4*>(dst + Lay<D>::off(row, 8 * ch)) = r[u];
    }
  }
};

// weight and gradient of one element with respect to the scaled score x = scale * q.k,
// from its raw score s, dpw = dP - delta (the dP product starts from -delta) and the
// row term lrow: P = exp2(t - lse2) and dS = P dpw dmod with dmod = d score_mod / dx.
//   soft-cap: t = cap2 tanh, tanh = 1 - 2 r with r = 1 / (e^{2x/cap} + 1), so
//             t - lse2 = lrow - 2 cap2 r with lrow = cap2 - lse2, and 1 - tanh^2 =
//             4 (r - r^2): dS is formed with r - r^2 and the factor 4 joins the scale
//   others:   t = score_log2(s), lrow = -lse2, dmod = 1
// The factor scale (times 4 for soft-cap) of dL/d(q.k) is applied once to dQ and dK.
// Computed for every pair; on blocks where some pair is outside the mask, mask_pair
// then zeroes both values of such pairs (a masked pair's values may be inf or NaN for
// an empty row and are discarded there).
template <int SCORE>
__device__ __forceinline__ void grad_elem(float s, float dpw, float lrow, const ScoreCtx& sc, int ig,
                                          int j, float& pv, float& ds) {
  if constexpr (SCORE == FA_S_SOFTCAP) {
    const float r = fast_rcp(fast_exp2(s * sc.capk) + 1.f);
    const float e = fast_exp2(__builtin_fmaf(-2.f * sc.cap2, r, lrow));
    pv = e;
    ds = e * dpw * __builtin_fmaf(-r, r, r);
  } else {
    const float e = fast_exp2(score_log2<SCORE>(s, sc, ig, j) + lrow);
    pv = e;
    ds = e * dpw;
  }
}

// the row term of grad_elem from a row's natural-log LSE
template <int SCORE>
__device__ __forceinline__ float grad_row_term(float lse, const ScoreCtx& sc) {
  return (SCORE == FA_S_SOFTCAP ? sc.cap2 : 0.f) - lse * kLog2e;
}

// the factor of dL/d(q.k) over the gradient grad_elem forms
template <int SCORE>
__device__ __forceinline__ float grad_scale(float scale) {
  return SCORE == FA_S_SOFTCAP ? 4.f * scale : scale;
}

// zero the weight and gradient of a pair outside the mask.  The empty asm keeps the
// compiler from sinking the pair's work into a branch on `ok`, which would serialize
// each pair behind its own exec mask.
__device__ __forceinline__ void mask_pair(bool ok, float& pv, float& ds) {
  asm volatile("" : "+v"(pv), "+v"(ds));
  pv = ok ? pv : 0.f;
  ds = ok ? ds : 0.f;
}

// ---- delta = rowsum(dO * O): D / 8 lanes per row, each with 16 bytes (8 values) of O
// and of dO per pass, the row's lanes reduced by xor shuffles inside their group; a
// workgroup takes kDeltaPasses groups of 256 / (D / 8) rows, all loads issued first
constexpr int kDeltaPasses = 4;
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams bp) {
  const FwdParams& p = bp.f;
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPP = 256 / LPR;      // rows per pass
  const int64_t rows = (int64_t)p.B * p.Hq * p.q_len;
  const int sub = threadIdx.x & (LPR - 1);
  const int64_t row0 = (int64_t)blockIdx.x * (RPP * kDeltaPasses) + threadIdx.x / LPR;
  u32x4 o[kDeltaPasses], g[kDeltaPasses];
#pragma unroll
  for (int k = 0; k < kDeltaPasses; ++k) {
    const int64_t row = min(row0 + (int64_t)k * RPP, rows - 1);   // clamped: out-of-range rows write nothing
    o[k] = load16(p.o + row * D + 8 * sub);
    g[k] = load16(bp.dout + row * D + 8 * sub);
  }
#pragma unroll
  for (int k = 0; k < kDeltaPasses; ++k) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += __builtin_bit_cast(float, o[k][e] << 16) * __builtin_bit_cast(float, g[k][e] << 16);
      acc += __builtin_bit_cast(float, o[k][e] & 0xffff0000u) * __builtin_bit_cast(float, g[k][e] & 0xffff0000u);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    const int64_t row = row0 + (int64_t)k * RPP;
    if (sub == 0 && row < rows) {
      bp.ndelta[row] = -acc;
      const float cap2 = p.score.kind == FA_S_SOFTCAP ? p.score.softcap * kLog2e : 0.f;   // as grad_row_term
      bp.lrow[row] = cap2 - p.lse[row] * kLog2e;
    }
  }
}

// A lane's pairs of one block as bits of a word: bit 4 m + rr for the position at offset
// 16 m + rr from the lane's first (the rows of its key in dK/dV, the keys of its row in
// dQ); the bits of positions at or past offset a.
__device__ __forceinline__ uint32_t ge_bits16(int a) {
  const int c = min(max(a, 0), 128);
  const int e0 = 4 * (c >> 4) + min(c & 15, 4);   // first pair at or past offset c
  return (uint32_t)(~0ull << e0);
}

// doc_bits of a lane: bit 4 m + e set when the document ID at ids[16 m + 4 g4 + e] (LDS)
// equals own, for m < n16 (one 4-ID group at a time: unrolled, the reads would be
// issued together and hold four times the registers)
__device__ __forceinline__ uint32_t doc_bits16(const int32_t* ids, int g4, int n16, int own) {
  uint32_t db = 0;
#pragma unroll 1
  for (int m = 0; m < n16; ++m) {
    const u32x4 d = *reinterpret_cast<const u32x4*>(ids + 16 * m + 4 * g4);
    uint32_t nib = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) nib |= (int)d[e] == own ? 1u << e : 0u;
    db |= nib << (4 * m);
  }
  return db;
}

// ---- dK, dV: one workgroup per (b, h_kv, KV block), NW = block_kv / 16 waves x 16 keys
// (the whole block shares each query block's Q and dO rows staged in LDS)
template <int D, int SCORE, int NW>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dkdv_kernel(BwdParams bp) {
  const FwdParams& p = bp.f;
  constexpr int NT = NW * 64;
  using L = Lay<D>;
  constexpr int RS = L::RS;
  constexpr int KS = D / 32;   // k-steps of the 16x16x32 products over the head dim
  constexpr int DT = D / 16;   // 16-row tiles of dK^T and dV^T
  constexpr int BQM = 128;     // largest query block
  // stored gradients, and rows copied HBM -> LDS into two buffers (128 KB): 128-key
  // blocks at d = 128 only
  constexpr bool kDs = NW == 8 && D == 128;
  constexpr bool kDma = kDs;
  constexpr int NB = kDma ? 2 : 1;
  // Q rows of one (head, block), then its dO rows
  __shared__ __attribute__((aligned(16))) uint8_t qg2[NB][2 * BQM * RS];
  __shared__ __attribute__((aligned(16))) float lse2[NB][BQM];         // row terms
  __shared__ __attribute__((aligned(16))) float del2[NB][BQM];         // -delta
  __shared__ __attribute__((aligned(16))) int32_t doc2[NB][BQM];       // document IDs of the rows

  // work item: (b, h_kv) fastest, then the KV block c ascending: every head's first
  // columns go out before any head's later ones (for causal-like rules the first columns
  // have the longest query-side lists), and consecutive (b, h_kv) spread over the XCDs
  const int item = blockIdx.x;
  const int nbh = p.B * p.Hkv;
  const int bh = item % nbh;
  const int c = item / nbh;
  const int hkv = bh % p.Hkv;
  const int b = bh / p.Hkv;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 15, g4 = lane >> 4;
  // the 8-element k-slice of lane group g4 in the S and dP products (the same for the
  // LDS-read and the register operand): groups 1 and 2 swapped. A probe of these 16-byte
  // row reads on the swizzled rows counted bank conflicts in half of their LDS cycles with
  // slice g4 and none with this order
  const int g4k = ((g4 & 1) << 1) | (g4 >> 1);
  const int q_len = (int)p.q_len, kv_len = (int)p.kv_len, bq = p.tab.bq;
  const int key0 = c * p.tab.bk + w * 16;   // first key of this wave
  const int j = key0 + col;                            // this lane's key (S column)

  // B operands: lane holds K[j][32 t + 8 g4 .. +8] and V[j][...] (rows past kv_len are
  // read clamped and masked)
  bf16x8 kf[KS], vf[KS];
  {
    const int jr = min(j, max(kv_len - 1, 0));
    const int64_t base = ((int64_t)(b * p.Hkv + hkv) * kv_len + jr) * D;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      kf[t] = __builtin_bit_cast(bf16x8, kv_len > 0 ? load16(p.k + base + 32 * t + 8 * g4k) : u32x4{0, 0, 0, 0});
      vf[t] = __builtin_bit_cast(bf16x8, kv_len > 0 ? load16(p.v + base + 32 * t + 8 * g4k) : u32x4{0, 0, 0, 0});
    }
  }
  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int32_t* docr = doc_row(p.doc, b);
  int doc_j = (p.prog.has_doc && j < kv_len) ? docr[j] : 0;
  // consumed here: first used inside the block loop, a load still counted as pending
  // there would make that use wait for the next block's prefetched rows too
  asm volatile("" : "+v"(doc_j));
  const int tb = p.tab.tB == 1 ? 0 : b;

  for (int hh = 0; hh < p.g; ++hh) {
    const int hq = hkv * p.g + hh;
    const ScoreCtx sc = make_score_ctx(p.score, p.scale, hq);
    const int th = p.tab.tH == 1 ? 0 : hq;
    const int line = (tb * p.tab.tH + th) * p.tab.nkb + c;   // q-side line of column c
    const int nf = uniform(p.tab.qfnum[line]);
    const int np = uniform(p.tab.qnum[line]);
    const int32_t* fl = p.tab.qfidx + uniform(p.tab.qfptr[line]);
    const int32_t* pl = p.tab.qidx + uniform(p.tab.qptr[line]);
    const int64_t bh = (int64_t)b * p.Hq + hq;
    const uint16_t* qsrc = p.q + bh * q_len * D;
    const uint16_t* gsrc = bp.dout + bh * q_len * D;
    const int n_ent = nf + np;
    // query block of list entry e and its row statistics (one per thread, bq <= 256)
    auto block_of = [&](int e) -> int { return load_uniform(e >= nf ? pl + (e - nf) : fl + e); };
    float nl2 = 0.f, ndl = 0.f;
    int ndc = 0;
    u32x4 pend_v = {0u, 0u, 0u, 0u};   // a gradient store held back (flush_pend)
    uint16_t* pend_p = nullptr;
    auto stats = [&](int r0) {
      const int i = r0 + (int)threadIdx.x;
      const bool ok = (int)threadIdx.x < bq && i < q_len;
      nl2 = ok ? bp.lrow[bh * q_len + i] : 0.f;
      ndl = ok ? bp.ndelta[bh * q_len + i] : 0.f;
      ndc = (ok && p.prog.has_doc) ? docr[i + p.q_offset] : 0;
    };
    // The steps of 32 query rows of one block (128-key blocks at d = 128), software
    // pipelined over scheduler-fenced stages. Stages 1-4 issue S and dP of step n over
    // k-steps t = 0..3 (four independent accumulators each), each from operands the
    // previous stage read, and read the transposed operands of step n - 1. Stage 5 forms
    // the weights and gradients of step n (VALU) with the dV and dK products of step n - 1
    // (MFMA, independent of that VALU) issued among them, so one wave's VALU and MFMA
    // overlap; it ends by reading step n + 1's first operands. The first step has no
    // previous products, and the block ends with those of its last step.
    auto pipelined = [&](int r0, const uint8_t* qs, const float* lse_s, const float* del_s,
                         uint32_t okw, bool sel, uint16_t* dst_tile) {
      const uint8_t* gs = qs + BQM * RS;   // one base: dO offsets become immediates
      // operands of k-step t for rows qn + 16 h + col: Q h0, dO h0, Q h1, dO h1
      auto rd1 = [&](int qn, int t, bf16x8 (&f)[4]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int off = L::off(qn + 16 * h + col, 32 * t + 8 * g4k);
          f[2 * h] = *reinterpret_cast<const bf16x8*>(qs + off);
          f[2 * h + 1] = *reinterpret_cast<const bf16x8*>(gs + off);
        }
      };
      // transposed dO and Q operands of head-dim tiles 2k and 2k + 1
      auto rd3 = [&](int q0, int k, bf16x8 (&f)[4]) {
        const int tr0 = q0 + 4 * g4 + (col >> 2);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int e = 16 * (2 * k + x) + 4 * (col & 3);
          f[2 * x] = cat_tr(gs + L::off(tr0, e), gs + L::off(tr0 + 16, e));
          f[2 * x + 1] = cat_tr(qs + L::off(tr0, e), qs + L::off(tr0 + 16, e));
        }
      };
      f32x4 s[2], dp[2], l4[2];
      bf16x8 pb, db;   // P and dS of the previous step: the B operands of its dV and dK
      bf16x8 n0[4], n1[4], f2[4], f3[4], p0[4], p1[4], p2[4], p3[4];
      auto mm1 = [&](const bf16x8 (&f)[4], int t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          s[h] = mma_k32(f[2 * h], kf[t], s[h]);
          dp[h] = mma_k32(f[2 * h + 1], vf[t], dp[h]);
        }
      };
      auto mm3 = [&](const bf16x8 (&f)[4], int k) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          dv[2 * k + x] = mma_k32(f[2 * x], pb, dv[2 * k + x]);
          dk[2 * k + x] = mma_k32(f[2 * x + 1], db, dk[2 * k + x]);
        }
      };
      auto sdp = [&](int q0, auto prev_c) {
        constexpr bool PREV = decltype(prev_c)::value;
        const int qp = q0 - 32;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[h] = *reinterpret_cast<const f32x4*>(del_s + q0 + 16 * h + 4 * g4);
          l4[h] = *reinterpret_cast<const f32x4*>(lse_s + q0 + 16 * h + 4 * g4);
        }
        mm1(n0, 0);
        rd1(q0, 2, f2);
        __builtin_amdgcn_sched_barrier(0);
        mm1(n1, 1);
        rd1(q0, 3, f3);
        __builtin_amdgcn_sched_barrier(0);
        mm1(f2, 2);
        if constexpr (PREV) rd3(qp, 0, p0);
        __builtin_amdgcn_sched_barrier(0);
        mm1(f3, 3);
        if constexpr (PREV) rd3(qp, 1, p1);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto grads = [&](int q0, auto prev_c) {
        constexpr bool PREV = decltype(prev_c)::value;
        float pv[8], ds[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int ig = r0 + q0 + 16 * h + 4 * g4 + rr + (int)p.q_offset;
            grad_elem<SCORE>(s[h][rr], dp[h][rr], l4[h][rr], sc, ig, j, pv[4 * h + rr], ds[4 * h + rr]);
          }
        }
        if constexpr (PREV) {
          mm3(p0, 0);
          mm3(p1, 1);
          rd3(q0 - 32, 2, p2);
          rd3(q0 - 32, 3, p3);
          mm3(p2, 2);
          mm3(p3, 3);
        }
        if (sel) {
#pragma unroll
          for (int x = 0; x < 8; ++x) mask_pair((okw >> (4 * (q0 >> 4) + x)) & 1u, pv[x], ds[x]);
        }
        pb = pack8(pv);
        db = pack8(ds);
        if (dst_tile && q0 + 32 < bq) {
          // 16 bytes per lane, 1 KB per wave, with the non-temporal policy (the tiles are
          // read once, by the dQ pass); the last step's part waits (pend)
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, db),
                                      reinterpret_cast<u32x4*>(dst_tile + (q0 >> 5) * (64 * 8)));
        }
        const int qn = min(q0 + 32, bq - 32);   // the last step reads its own rows again
        rd1(qn, 0, n0);
        rd1(qn, 1, n1);
        __builtin_amdgcn_sched_barrier(0);
      };
      rd1(0, 0, n0);
      rd1(0, 1, n1);
      __builtin_amdgcn_sched_barrier(0);
      sdp(0, std::false_type{});
      grads(0, std::false_type{});
      for (int q0 = 32; q0 < bq; q0 += 32) {
        sdp(q0, std::true_type{});
        grads(q0, std::true_type{});
      }
      // the last step's dV and dK
      const int ql = bq - 32;
      rd3(ql, 0, p0);
      rd3(ql, 1, p1);
      __builtin_amdgcn_sched_barrier(0);
      mm3(p0, 0);
      rd3(ql, 2, p2);
      __builtin_amdgcn_sched_barrier(0);
      mm3(p1, 1);
      rd3(ql, 3, p3);
      __builtin_amdgcn_sched_barrier(0);
      mm3(p2, 2);
      mm3(p3, 3);
      __builtin_amdgcn_sched_barrier(0);
      if (dst_tile) {
        pend_v = __builtin_bit_cast(u32x4, db);
        pend_p = dst_tile + ((bq - 32) >> 5) * (64 * 8);
      }
    };
    // the block of list entry e, rows r0.., from the staged rows, row terms, -delta and
    // document IDs
    auto compute = [&](int e, int r0, const uint8_t* qs, const uint8_t* gs, const float* lse_s,
                       const float* del_s, const int32_t* doc_s, uint16_t* dst_tile) {
      const bool part = e >= nf;
      // which of the lane's 32 rows (r0 + 16 m + 4 g4 + rr) may see key j: the row
      // bounds, and on partial blocks the mask program over the whole group
      const int rb = r0 + 4 * g4 + (int)p.q_offset;
      auto span = [&](int lo, int hi) -> uint32_t { return ge_bits16(lo - rb) & ~ge_bits16(hi - rb + 1); };
      uint32_t okw = j < kv_len ? span((int)p.q_offset, (int)p.q_offset + q_len - 1) : 0u;
      if (part) {
        const uint32_t db = p.prog.has_doc ? doc_bits16(doc_s, g4, bq >> 4, doc_j) : 0u;
        okw &= mask_word(p.prog, [&](int op, int a) { return col_leaf(op, a, j, span, db); });
      }
      // pairs outside the mask are zeroed only on blocks where the wave has some
      const bool sel = __ballot(okw != 0xffffffffu) != 0;
      if constexpr (kDma) {
        pipelined(r0, qs, lse_s, del_s, okw, sel, dst_tile);
        return;
      }
      for (int q0 = 0; q0 < bq; q0 += 32) {
        // S and dP (16 rows x 16 keys each) of rows q0 + 16 h + (0..15), h = 0, 1, on
        // 16x16x32 tiles over the head dim
        // (lane: rows q0 + 16 h + 4 g4 + rr, key j; the rows' terms and -delta as one
        // 16-byte LDS word each per h; dP starts from -delta)
        f32x4 s[2], dp[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[h] = *reinterpret_cast<const f32x4*>(del_s + q0 + 16 * h + 4 * g4);
#pragma unroll
          for (int t = 0; t < KS; ++t) {
            const int off = L::off(q0 + 16 * h + col, 32 * t + 8 * g4k);
            s[h] = mma_k32(*reinterpret_cast<const bf16x8*>(qs + off), kf[t], s[h]);
            dp[h] = mma_k32(*reinterpret_cast<const bf16x8*>(gs + off), vf[t], dp[h]);
          }
        }
        float pv[8], ds[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + q0 + 16 * h + 4 * g4);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int xr = q0 + 16 * h + 4 * g4 + rr;
            const int ig = r0 + xr + (int)p.q_offset;
            grad_elem<SCORE>(s[h][rr], dp[h][rr], l4[rr], sc, ig, j, pv[4 * h + rr], ds[4 * h + rr]);
          }
        }
        if (sel) {
#pragma unroll
          for (int x = 0; x < 8; ++x) mask_pair((okw >> (4 * (q0 >> 4) + x)) & 1u, pv[x], ds[x]);
        }
        const bf16x8 pb = pack8(pv), db = pack8(ds);
        if (kDs && dst_tile) {
          // 16 bytes per lane, 1 KB per wave, with the non-temporal policy (the tiles are
          // read once, by the dQ pass)
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, db),
                                      reinterpret_cast<u32x4*>(dst_tile + (q0 >> 5) * (64 * 8)));
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the 32 rows (16x16x32): the lane holds P
        // and dS in the contraction order of cat_tr (rows q0 + 4 g4 + e, then q0 + 16 +
        // 4 g4 + e), and the A operands (head dim x rows) come from transposing reads
        const int tr0 = q0 + 4 * g4 + (col >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int e = 16 * dt + 4 * (col & 3);
          dv[dt] = mma_k32(cat_tr(gs + L::off(tr0, e), gs + L::off(tr0 + 16, e)), pb, dv[dt]);
          dk[dt] = mma_k32(cat_tr(qs + L::off(tr0, e), qs + L::off(tr0 + 16, e)), db, dk[dt]);
        }
      }
    };
    // the block's stored-gradient tile, (r, c) of the head's NQB x NKB grid of tiles, in
    // the order of the lanes that form it (BwdParams::ds); the wave's part
    auto tile_of = [&](int rblk) -> uint16_t* {
      if (!(kDs && bp.ds && rblk < p.tab.nqb)) return nullptr;
      const int64_t slot = (bh * p.tab.nqb + rblk) * p.tab.nkb + c;
      return bp.ds + slot * (128 * 128) + w * (4 * 64 * 8) + lane * 8;
    };
    // the previous block's last gradient store, held until the next block's wait so that
    // the wait does not wait for it
    auto flush_pend = [&]() {
      if (pend_p) {
        __builtin_nontemporal_store(pend_v, reinterpret_cast<u32x4*>(pend_p));
        pend_p = nullptr;
      }
    };
    auto put_stats = [&](int buf) {
      if ((int)threadIdx.x < bq) {
        lse2[buf][threadIdx.x] = nl2;
        del2[buf][threadIdx.x] = ndl;
        doc2[buf][threadIdx.x] = ndc;
      }
    };
    if constexpr (kDma) {
      // Entry e's block lands in buffer e & 1 by LDS-DMA issued one block ahead: its Q
      // and dO rows, row terms, -delta and document IDs (rows past the end repeat the
      // last row; their pairs are masked). No staging registers and no load the compiler
      // sees, so one explicit wait and one barrier per block publish it.
      auto copy_rows = [&](int r0, int buf) {
        const uint16_t* qb = qsrc + (int64_t)r0 * D;
        const uint16_t* gb = gsrc + (int64_t)r0 * D;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int row = 16 * w + 4 * u;   // the instruction's first row (wave-uniform)
          if (row < bq) {
            // lane l fills 16-byte slot l & 15 of row row + (l >> 4): the chunk that
            // Lay's swizzle puts there; rows past the end repeat the last row (masked)
            const int rl = row + (lane >> 4);
            const int rg = min(r0 + rl, q_len - 1) - r0;
            const int lc = (lane & 15) ^ (2 * (rl & 7) + ((rl >> 3) & 1));
            const uint32_t voff = (uint32_t)(rg * (D * 2) + lc * 16);
            dma16_s<0>(lds_addr(qg2[buf]) + row * RS, qb, voff);
            dma16_s<0>(lds_addr(qg2[buf]) + (BQM + row) * RS, gb, voff);
          }
        }
        // waves 0, 1, 2: row terms, -delta, document IDs, 64 rows of 4 bytes per copy
        if (w < (p.prog.has_doc ? 3 : 2)) {
          const int32_t* src = w == 0 ? reinterpret_cast<const int32_t*>(bp.lrow + bh * q_len)
                             : w == 1 ? reinterpret_cast<const int32_t*>(bp.ndelta + bh * q_len)
                                      : docr + p.q_offset;
          const uint32_t dst = w == 0 ? lds_addr(lse2[buf]) : w == 1 ? lds_addr(del2[buf]) : lds_addr(doc2[buf]);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if (64 * u < bq) {
              const int rg = min(r0 + 64 * u + lane, q_len - 1);
              dma4_s(dst + 256 * u, src, (uint32_t)(rg * 4));
            }
          }
        }
      };
      __syncthreads();   // the previous head's last block is consumed in every wave
      if (n_ent > 0) copy_rows(block_of(0) * bq, 0);
      for (int e = 0; e < n_ent; ++e) {
        const int rblk = block_of(e), cur = e & 1;
        wait_dma();        // this block's copies (and every earlier store) have landed
        __syncthreads();   // in every wave; the other buffers' block is consumed
        if (e + 1 < n_ent) copy_rows(block_of(e + 1) * bq, cur ^ 1);
        flush_pend();      // after the wait: it completes during this block
        compute(e, rblk * bq, qg2[cur], qg2[cur] + BQM * RS, lse2[cur], del2[cur], doc2[cur], tile_of(rblk));
      }
      flush_pend();
    } else {
      RowStage<D, NT> sq, sg;
      if (n_ent > 0) {
        const int r0n = block_of(0) * bq;
        sq.fetch(qsrc, r0n, bq, q_len);
        sg.fetch(gsrc, r0n, bq, q_len);
        stats(r0n);
      }
      for (int e = 0; e < n_ent; ++e) {
        const int rblk = block_of(e);
        __syncthreads();   // the previous block's rows are consumed
        sq.put(qg2[0], bq);
        sg.put(qg2[0] + BQM * RS, bq);
        put_stats(0);
        __syncthreads();
        if (e + 1 < n_ent) {   // next block's rows travel while this one is computed
          const int r0n = block_of(e + 1) * bq;
          sq.fetch(qsrc, r0n, bq, q_len);
          sg.fetch(gsrc, r0n, bq, q_len);
          stats(r0n);
        }
        compute(e, rblk * bq, qg2[0], qg2[0] + BQM * RS, lse2[0], del2[0], doc2[0], tile_of(rblk));
      }
    }
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] *= grad_scale<SCORE>(p.scale);
  // lane holds key j, head dims 16 dt + 4 g4 .. +4
  if (j < kv_len) {
    const int64_t base = ((int64_t)(b * p.Hkv + hkv) * kv_len + j) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      *reinterpret_cast<f32x4*>(bp.dk + base + 16 * dt + 4 * g4) = dk[dt];
      *reinterpret_cast<f32x4*>(bp.dv + base + 16 * dt + 4 * g4) = dv[dt];
    }
  }
}

// ---- dQ: one workgroup per (b, h_q, query block), NW waves x 16 rows
template <int D, int SCORE, int NW>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(BwdParams bp) {
  const FwdParams& p = bp.f;
  constexpr int NT = NW * 64;
  using L = Lay<D>;
  constexpr int RS = L::RS;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int BKM = 128;
  __shared__ __attribute__((aligned(16))) uint8_t ks[BKM * RS];
  __shared__ __attribute__((aligned(16))) uint8_t vs[BKM * RS];
  __shared__ __attribute__((aligned(16))) int32_t doc_s[BKM];   // document IDs of the keys
  // gradient of the position table: one bin per offset of this query head
  constexpr int kBins = SCORE == FA_S_RELPOS ? 2 * kRelGradMaxRadius + 1 : 1;
  __shared__ float bins_s[kBins];

  // work item: (b, h_q) and the rank-th longest query block of its table entry (the
  // forward's order: the tables' work order when present, else descending index)
  const int nqb = p.tab.nqb;
  const int nbh = p.B * p.Hq;
  const int rank = blockIdx.x / nbh;
  const int bh = blockIdx.x - rank * nbh;   // b * Hq + h_q
  const int b = bh / p.Hq, hq = bh - b * p.Hq, hkv = hq / p.g;
  const int tb = p.tab.tB == 1 ? 0 : b;
  const int th = p.tab.tH == 1 ? 0 : hq;
  const int r = p.tab.order ? uniform(p.tab.order[(tb * p.tab.tH + th) * nqb + rank]) : nqb - 1 - rank;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 15, g4 = lane >> 4;
  // the 8-element k-slice of lane group g4 in the S and dP products (the same for the
  // LDS-read and the register operand): groups 1 and 2 swapped. A probe of these 16-byte
  // row reads on the swizzled rows counted bank conflicts in half of their LDS cycles with
  // slice g4 and none with this order
  const int g4k = ((g4 & 1) << 1) | (g4 >> 1);
  const int q_len = (int)p.q_len, kv_len = (int)p.kv_len, bk = p.tab.bk;
  const int i = r * p.tab.bq + w * 16 + col;   // this lane's row (S^T column)
  const bool row_ok = i < q_len;
  const int ig = i + (int)p.q_offset;

  // B operands: Q[i][32 t + 8 g4 .. +8] and dO[i][...]
  bf16x8 qf[KS], gf[KS];
  {
    const int ir = min(i, q_len - 1);
    const int64_t base = ((int64_t)bh * q_len + ir) * D;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      qf[t] = __builtin_bit_cast(bf16x8, load16(p.q + base + 32 * t + 8 * g4k));
      gf[t] = __builtin_bit_cast(bf16x8, load16(bp.dout + base + 32 * t + 8 * g4k));
    }
  }
  const ScoreCtx sc = make_score_ctx(p.score, p.scale, hq);
  const float lrow = row_ok ? bp.lrow[(int64_t)bh * q_len + i] : 0.f;
  const float ndelta = row_ok ? bp.ndelta[(int64_t)bh * q_len + i] : 0.f;
  const f32x4 dp0 = f32x4{ndelta, ndelta, ndelta, ndelta};   // dP^T starts from -delta
  const int32_t* docr = doc_row(p.doc, b);
  int doc_i = (p.prog.has_doc && row_ok) ? docr[ig] : 0;
  asm volatile("" : "+v"(doc_i));   // (as doc_j in the dK/dV kernel)
  f32x4 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // score_mod parameter gradients: dL/ds' = dS per pair (ALiBi and the position table
  // add to the scaled score, dmod = 1), with ds'/d slope = j - i (ALiBi) and
  // ds'/d table[h][clip(i - j) + R] = 1; saturated offsets collect in registers, the
  // others in LDS bins
  const bool want_slope = SCORE == FA_S_ALIBI && bp.dslopes != nullptr;
  const bool want_table = SCORE == FA_S_RELPOS && bp.dtable != nullptr;
  const int R = p.score.radius;
  float g_slope = 0.f, g_far = 0.f, g_ahead = 0.f;
  if (want_table) {
    for (int x = threadIdx.x; x < 2 * R + 1; x += NT) bins_s[x] = 0.f;
    __syncthreads();   // (kernel argument: uniform) bins clear before any add
  }

  const int row = (tb * p.tab.tH + th) * nqb + r;
  const int nf = uniform(p.tab.fnum[row]);
  const int np = uniform(p.tab.num[row]);
  const int32_t* fl = p.tab.fidx + uniform(p.tab.fptr[row]);
  const int32_t* pl = p.tab.idx + uniform(p.tab.ptr[row]);
  const int64_t kvh = (int64_t)(b * p.Hkv + hkv) * kv_len;
  const int n_ent = nf + np;
  auto block_of = [&](int e) -> int { return load_uniform(e >= nf ? pl + (e - nf) : fl + e); };
  RowStage<D, NT> sk, sv;
  // document ID of key j0 + threadIdx.x (threads below bk; keys past kv_len read the last)
  auto key_doc = [&](int j0) -> int {
    return (p.prog.has_doc && (int)threadIdx.x < bk) ? docr[min(j0 + (int)threadIdx.x, kv_len - 1)] : 0;
  };
  int ndc = 0;
  if (n_ent > 0) {
    sk.fetch(p.k + kvh * D, block_of(0) * bk, bk, kv_len);
    sv.fetch(p.v + kvh * D, block_of(0) * bk, bk, kv_len);
    ndc = key_doc(block_of(0) * bk);
  }
  for (int e = 0; e < n_ent; ++e) {
    const bool part = e >= nf;
    const int j0 = block_of(e) * bk;
    __syncthreads();
    sk.put(ks, bk);
    sv.put(vs, bk);
    if ((int)threadIdx.x < bk) doc_s[threadIdx.x] = ndc;
    __syncthreads();
    if (e + 1 < n_ent) {   // next block's K and V travel while this one is computed
      sk.fetch(p.k + kvh * D, block_of(e + 1) * bk, bk, kv_len);
      sv.fetch(p.v + kvh * D, block_of(e + 1) * bk, bk, kv_len);
      ndc = key_doc(block_of(e + 1) * bk);
    }
    // which of the lane's 32 keys (j0 + 16 m + 4 g4 + rr) row i may see: the key
    // bounds, and on partial blocks the mask program over the whole group
    const int kb = j0 + 4 * g4;
    auto span = [&](int lo, int hi) -> uint32_t { return ge_bits16(lo - kb) & ~ge_bits16(hi - kb + 1); };
    uint32_t okw = row_ok ? span(0, kv_len - 1) : 0u;
    if (part) {
      const uint32_t db = p.prog.has_doc ? doc_bits16(doc_s, g4, bk >> 4, doc_i) : 0u;
      okw &= mask_word(p.prog, [&](int op, int a) { return row_leaf(op, a, ig, span, db); });
    }
    // pairs outside the mask are zeroed only on blocks where the wave has some
    const bool sel = __ballot(okw != 0xffffffffu) != 0;
    // lane: keys j0 + k0 + 16 h + 4 g4 + rr, row i: weights and gradients of the 32
    // keys from S^T and dP^T, the parameter gradients, and dS^T as the B operand db
    auto grads = [&](int k0, const f32x4 (&s)[2], const f32x4 (&dp)[2]) -> bf16x8 {
      // lane: keys j0 + k0 + 16 h + 4 g4 + rr, row i
      float pv[8], ds[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          grad_elem<SCORE>(s[h][rr], dp[h][rr], lrow, sc, ig, j0 + k0 + 16 * h + 4 * g4 + rr, pv[4 * h + rr],
                           ds[4 * h + rr]);
      if (sel) {
#pragma unroll
        for (int x = 0; x < 8; ++x) mask_pair((okw >> (4 * (k0 >> 4) + x)) & 1u, pv[x], ds[x]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int jj = j0 + k0 + 16 * h + 4 * g4 + rr;
          const float d = ds[4 * h + rr];
          if constexpr (SCORE == FA_S_ALIBI) {
            if (want_slope) g_slope = __builtin_fmaf(d, (float)(jj - ig), g_slope);
          }
          if constexpr (SCORE == FA_S_RELPOS) {
            if (want_table && d != 0.f) {
              const int rel = ig - jj;
              if (rel >= R) g_far += d;
              else if (rel <= -R) g_ahead += d;
              else unsafeAtomicAdd(&bins_s[rel + R], d);
            }
          }
        }
      (void)pv;
      return pack8(ds);
    };
    if constexpr (D == 128 && NW == 8) {
      // 128-dim heads, 128-row query blocks: each 32-key step is software-pipelined over
      // scheduler-fenced stages whose products use LDS operands the previous stage read
      // (S^T and dP^T over k-steps 0..3, then the gradients, then dQ^T over head-dim
      // tiles 0..3 and 4..7, which read the next step's first operands)
      auto rd_s = [&](int kn, int t, bf16x8 (&f)[4]) {   // K h0, V h0, K h1, V h1
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int off = L::off(kn + 16 * h + col, 32 * t + 8 * g4k);
          f[2 * h] = *reinterpret_cast<const bf16x8*>(ks + off);
          f[2 * h + 1] = *reinterpret_cast<const bf16x8*>(vs + off);
        }
      };
      auto rd_q = [&](int k0, int grp, bf16x8 (&f)[4]) {   // K^T tiles 4 grp .. + 3
        const int tr0 = k0 + 4 * g4 + (col >> 2);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int e = 16 * (4 * grp + x) + 4 * (col & 3);
          f[x] = cat_tr(ks + L::off(tr0, e), ks + L::off(tr0 + 16, e));
        }
      };
      bf16x8 n0[4], n1[4];
      rd_s(0, 0, n0);
      rd_s(0, 1, n1);
      __builtin_amdgcn_sched_barrier(0);
      for (int k0 = 0; k0 < bk; k0 += 32) {
        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}, dp[2] = {dp0, dp0};
        bf16x8 f2[4], f3[4], a0[4], a1[4];
        auto mm_s = [&](const bf16x8 (&f)[4], int t) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            s[h] = mma_k32(f[2 * h], qf[t], s[h]);
            dp[h] = mma_k32(f[2 * h + 1], gf[t], dp[h]);
          }
        };
        mm_s(n0, 0);
        rd_s(k0, 2, f2);
        __builtin_amdgcn_sched_barrier(0);
        mm_s(n1, 1);
        rd_s(k0, 3, f3);
        __builtin_amdgcn_sched_barrier(0);
        mm_s(f2, 2);
        rd_q(k0, 0, a0);
        __builtin_amdgcn_sched_barrier(0);
        mm_s(f3, 3);
        rd_q(k0, 1, a1);
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 db = grads(k0, s, dp);
        __builtin_amdgcn_sched_barrier(0);
        const int kn = min(k0 + 32, bk - 32);   // the last step reads its own keys again
#pragma unroll
        for (int x = 0; x < 4; ++x) dq[x] = mma_k32(a0[x], db, dq[x]);
        rd_s(kn, 0, n0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 4; ++x) dq[4 + x] = mma_k32(a1[x], db, dq[4 + x]);
        rd_s(kn, 1, n1);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for (int k0 = 0; k0 < bk; k0 += 32) {
        f32x4 s[2], dp[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[h] = dp0;
#pragma unroll
          for (int t = 0; t < KS; ++t) {
            const int off = L::off(k0 + 16 * h + col, 32 * t + 8 * g4k);
            s[h] = mma_k32(*reinterpret_cast<const bf16x8*>(ks + off), qf[t], s[h]);
            dp[h] = mma_k32(*reinterpret_cast<const bf16x8*>(vs + off), gf[t], dp[h]);
          }
        }
        const bf16x8 db = grads(k0, s, dp);
        // dQ^T += K^T dS^T over the 32 keys (16x16x32; contraction order as in cat_tr)
        const int tr0 = k0 + 4 * g4 + (col >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int e = 16 * dt + 4 * (col & 3);
          dq[dt] = mma_k32(cat_tr(ks + L::off(tr0, e), ks + L::off(tr0 + 16, e)), db, dq[dt]);
        }
      }
    }
  }
  // parameter gradients: wave sums, then one global add per wave (slopes) or per bin
  if (want_slope) {
    for (int off = 32; off > 0; off >>= 1) g_slope += __shfl_xor(g_slope, off);
    if ((threadIdx.x & 63) == 0) unsafeAtomicAdd(&bp.dslopes[hq], g_slope);
  }
  if (want_table) {
    for (int off = 32; off > 0; off >>= 1) {
      g_far += __shfl_xor(g_far, off);
      g_ahead += __shfl_xor(g_ahead, off);
    }
    if ((threadIdx.x & 63) == 0) {
      unsafeAtomicAdd(&bins_s[2 * R], g_far);
      unsafeAtomicAdd(&bins_s[0], g_ahead);
    }
    __syncthreads();
    float* gt = bp.dtable + (int64_t)hq * (2 * R + 1);
    for (int x = threadIdx.x; x < 2 * R + 1; x += NT) {
      const float v = bins_s[x];
      if (v != 0.f) unsafeAtomicAdd(&gt[x], v);
    }
  }
  if (row_ok) {
    float* out = bp.dq + ((int64_t)bh * q_len + i) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(out + 16 * dt + 4 * g4) = dq[dt] * grad_scale<SCORE>(p.scale);
  }
}

// ---- dQ from the gradients stored by the dK/dV pass (128 x 128 blocks, D = 128): one
// workgroup per (b, h_q, query block), one wave per 16 rows.  For each listed KV block
// its K rows and its stored tile (rows are the block's keys, 128 values each: the same
// 256-byte rows as K) go to LDS, and dQ^T += K^T dS^T over 32 keys at a time takes both
// operands from transposing reads.  No score is recomputed.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_ds_kernel(BwdParams bp) {
  static_assert(D == 128 && NW == 8, "stored gradient tiles are read for 128 x 128 blocks at d = 128");
  const FwdParams& p = bp.f;
  constexpr int NT = NW * 64;
  using L = Lay<D>;
  constexpr int RS = L::RS;
  constexpr int DT = D / 16;
  constexpr int BKM = 128;
  __shared__ __attribute__((aligned(16))) uint8_t ks[BKM * RS];
  __shared__ __attribute__((aligned(16))) uint8_t ts[BKM * RS];   // the stored tile

  // work item as in bwd_dq_kernel
  const int nqb = p.tab.nqb;
  const int nbh = p.B * p.Hq;
  const int rank = blockIdx.x / nbh;
  const int bh = blockIdx.x - rank * nbh;
  const int b = bh / p.Hq, hq = bh - b * p.Hq, hkv = hq / p.g;
  const int tb = p.tab.tB == 1 ? 0 : b;
  const int th = p.tab.tH == 1 ? 0 : hq;
  const int r = p.tab.order ? uniform(p.tab.order[(tb * p.tab.tH + th) * nqb + rank]) : nqb - 1 - rank;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 15, g4 = lane >> 4;
  const int q_len = (int)p.q_len, kv_len = (int)p.kv_len, bk = p.tab.bk;
  const int i = r * p.tab.bq + w * 16 + col;
  f32x4 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int g0 = (tb * p.tab.tH + th) * nqb;
  const int row = g0 + r;
  const int nf = uniform(p.tab.fnum[row]);
  const int np = uniform(p.tab.num[row]);
  const int32_t* fl = p.tab.fidx + uniform(p.tab.fptr[row]);
  const int32_t* pl = p.tab.idx + uniform(p.tab.ptr[row]);
  const int64_t kvh = (int64_t)(b * p.Hkv + hkv) * kv_len;
  // the row's tiles: (r, c) of the head's NQB x NKB grid
  const uint16_t* tiles = bp.ds + ((int64_t)bh * nqb + r) * p.tab.nkb * (BKM * BKM);
  const int n_ent = nf + np;
  auto block_of = [&](int e) -> int { return load_uniform(e >= nf ? pl + (e - nf) : fl + e); };
  RowStage<D, NT> sk, st;
  auto fetch = [&](int e) {
    const int c = block_of(e);
    sk.fetch(p.k + kvh * D, c * bk, bk, kv_len);
    // the tile: 32 KB read once, with the non-temporal policy (streaming reads run at
    // about 7 TB/s with it, 5.2 TB/s without)
    const u32x4* t = reinterpret_cast<const u32x4*>(tiles + (int64_t)c * (BKM * BKM));
#pragma unroll
    for (int u = 0; u < RowStage<D, NT>::PER; ++u) st.r[u] = __builtin_nontemporal_load(t + threadIdx.x + u * NT);
  };
  if (n_ent > 0) fetch(0);
  for (int e = 0; e < n_ent; ++e) {
    __syncthreads();
    sk.put(ks, bk);
    // the tile's 16-byte chunk x (BwdParams::ds) holds key 16 (x >> 8) + (x & 15) for
    // rows 32 ((x >> 6) & 3) + 4 ((x >> 4) & 3) + (0..3), then for those rows + 16
#pragma unroll
    for (int u = 0; u < RowStage<D, NT>::PER; ++u) {
      const int x = threadIdx.x + u * NT;
      const int key = 16 * (x >> 8) + (x & 15);
      const int rw = 32 * ((x >> 6) & 3) + 4 * ((x >> 4) & 3);
      *reinterpret_cast<u32x2*>(ts + L::off(key, rw)) = u32x2{st.r[u][0], st.r[u][1]};
      *reinterpret_cast<u32x2*>(ts + L::off(key, rw + 16)) = u32x2{st.r[u][2], st.r[u][3]};
    }
    __syncthreads();
    if (e + 1 < n_ent) fetch(e + 1);   // the next block travels while this one is used
    // 32 products per block: key step k = i / 8 (32 keys), head-dim tile i % 8. Each
    // product's A operand is read two products ahead and the next key step's B operand
    // three ahead, one scheduler-fenced product at a time, so the LDS latency runs under
    // the MFMAs.
    // B of key step k: the stored gradients of rows 16 w + col for keys 32 k + 4 g4 +
    // (0..3) and 32 k + 16 + 4 g4 + (0..3), the contraction order of cat_tr
    auto rd_b = [&](int k) {
      const int kr = 32 * k + 4 * g4 + (col >> 2);
      const int ro = 16 * w + 4 * (col & 3);
      return cat_tr(ts + L::off(kr, ro), ts + L::off(kr + 16, ro));
    };
    auto rd_a = [&](int i) {
      const int kr = 32 * (i >> 3) + 4 * g4 + (col >> 2);
      const int ee = 16 * (i & 7) + 4 * (col & 3);
      return cat_tr(ks + L::off(kr, ee), ks + L::off(kr + 16, ee));
    };
    bf16x8 a0 = rd_a(0), a1 = rd_a(1), b0 = rd_b(0), b1 = b0;
    __builtin_amdgcn_sched_barrier(0);
    static_for<4 * DT>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      bf16x8 a2 = a1;
      if constexpr (i + 2 < 4 * DT) a2 = rd_a(i + 2);
      if constexpr ((i & 7) == 5 && i + 3 < 4 * DT) b1 = rd_b((i >> 3) + 1);
      dq[i & 7] = mma_k32(a0, b0, dq[i & 7]);
      a0 = a1;
      a1 = a2;
      if constexpr ((i & 7) == 7) b0 = b1;
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  if (i < q_len) {
    const float gs = p.score.kind == FA_S_SOFTCAP ? 4.f * p.scale : p.scale;   // as grad_scale
    float* out = bp.dq + ((int64_t)bh * q_len + i) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(out + 16 * dt + 4 * g4) = dq[dt] * gs;
  }
}

// clears a parameter-gradient output before the dQ pass adds into it (a kernel, not a
// memset, so the work stays an ordinary launch on the caller's stream)
__global__ __launch_bounds__(256) void zero_kernel(float* x, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n) x[t] = 0.f;
}

template <int D, int SCORE>
hipError_t launch_bwd_score(const BwdParams& bp, hipStream_t s) {
  const FwdParams& p = bp.f;
  const int64_t items = (int64_t)p.B * p.Hkv * p.tab.nkb;
  if (items > 0) {
    if (p.tab.bk == 128) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, SCORE, 8>), dim3((unsigned)items), dim3(512), 0, s, bp);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, SCORE, 4>), dim3((unsigned)items), dim3(256), 0, s, bp);
    }
  }
  const int64_t qitems = (int64_t)p.B * p.Hq * p.tab.nqb;
  float* pg = SCORE == FA_S_ALIBI ? bp.dslopes : (SCORE == FA_S_RELPOS ? bp.dtable : nullptr);
  if (pg != nullptr) {
    const int64_t n = SCORE == FA_S_ALIBI ? (int64_t)p.Hq : (int64_t)p.Hq * (2 * p.score.radius + 1);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, pg, n);
  }
  if (qitems > 0) {
    if constexpr (D == 128) {
      if (bp.ds) {   // the host enables stored gradients for 128 x 128 blocks only
        hipLaunchKernelGGL((bwd_dq_ds_kernel<128, 8>), dim3((unsigned)qitems), dim3(512), 0, s, bp);
        return hipGetLastError();
      }
    }
    if (p.tab.bq == 128) {
      hipLaunchKernelGGL((bwd_dq_kernel<D, SCORE, 8>), dim3((unsigned)qitems), dim3(512), 0, s, bp);
    } else {
      hipLaunchKernelGGL((bwd_dq_kernel<D, SCORE, 4>), dim3((unsigned)qitems), dim3(256), 0, s, bp);
    }
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& bp, hipStream_t s) {
  const FwdParams& p = bp.f;
  const int64_t rows = (int64_t)p.B * p.Hq * p.q_len;
  constexpr int64_t kDeltaRows = 256 / (D / 8) * kDeltaPasses;   // rows per workgroup
  if (rows > 0) hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + kDeltaRows - 1) / kDeltaRows)), dim3(256), 0, s, bp);
  switch (p.score.kind) {
    case FA_S_IDENTITY: return launch_bwd_score<D, FA_S_IDENTITY>(bp, s);
    case FA_S_ALIBI: return launch_bwd_score<D, FA_S_ALIBI>(bp, s);
    case FA_S_SOFTCAP: return launch_bwd_score<D, FA_S_SOFTCAP>(bp, s);
    default: return launch_bwd_score<D, FA_S_RELPOS>(bp, s);
  }
}

}  // namespace

size_t backward_workspace_min_bytes(const FwdParams& p) {
  // -delta, then the row terms, each from a 256-byte boundary
  return 2 * (((size_t)p.B * p.Hq * p.q_len * sizeof(float) + 255) & ~(size_t)255);
}

size_t backward_ds_bytes(const FwdParams& p, bool param_grads) {
  if (param_grads || p.d != 128 || p.tab.bq != 128 || p.tab.bk != 128) return 0;
  const size_t bytes = (size_t)p.B * p.Hq * p.tab.nqb * p.tab.nkb * 128 * 128 * sizeof(uint16_t);
  return bytes <= kDsMaxBytes ? bytes : 0;
}

hipError_t launch_backward(const BwdParams& bp, hipStream_t s) {
  return bp.f.d == 128 ? launch_bwd_d<128>(bp, s) : launch_bwd_d<64>(bp, s);
}

}  // namespace fa
