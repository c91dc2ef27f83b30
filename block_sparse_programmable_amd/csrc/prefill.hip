// Block-sparse attention forward, prefill shape (many query rows), for gfx950.
//
// One workgroup owns one query block (b, h_q, r) and walks the KV blocks that the
// block table lists for its row: first the FULL list, then the PARTIAL list
// ("FlexAttention: compiler optimization of custom attention", section 3 -- the
// forward fixes a query tile, reads the KV block numbers from the BlockMask and, for
// each kept block, computes Q K^T * scale, applies score_mod, applies mask_mod only
// on partial blocks, then updates the online softmax and accumulates with V).
// Online softmax state and merge law: "Kernels: turning logical sparsity into real
// speed", section 3; "Flash Attention self-test answers", Q24-Q29.  Skipping blocks
// and masking before the row statistics: "FlexAttention: from rules to fused
// kernels", section 3.1.
//
// gfx950 mapping
//   * waves: NW = block_q / 32; wave w owns 32 query rows.  Scores are computed
//     transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so that every lane holds
//     one query row (column) and 16 keys per 32-key tile: row max / row sum stay in
//     the lane apart from one exchange between the two 32-lane halves.
//   * O is accumulated transposed as well (O^T = V^T P^T): P^T in the MFMA output
//     layout feeds the B operand directly once the key order inside each 16-key step
//     is permuted; V^T is stored in LDS with the same permutation.
//   * KV is staged in 64-key sub-tiles: K row-major and V transposed in LDS, 16-byte
//     chunks XOR-swizzled by row so that ds_read_b128 fragment reads are bank-conflict
//     free; global loads are 16 bytes per lane and cover whole 256-byte rows per
//     quarter-wave.  Two LDS buffers plus register staging give one barrier per
//     sub-tile with the next sub-tile's loads in flight during compute.
//   * softmax runs in base 2.  Where score_mod is monotone in the raw score (identity,
//     soft-cap, a saturated relative-position bias) the row maximum is taken on the raw
//     MFMA output and mapped once per row; the scale folds into the FMA feeding exp2.
//   * the running maximum is refreshed only when a row's tile maximum exceeds it by
//     more than 2^8 (in base 2), so the O rescale is rare; the normaliser and O use the
//     same reference, which keeps the result exact while bounding every weight by 2^8.
//   * partial blocks: the mask rule is pre-compiled on the host into a per-row key
//     interval (intersections of causal / window / prefix) plus an optional document
//     compare against IDs staged in LDS; other programs use the generic interpreter.
//   * grid order: longest rows first (query block index descending), and heads
//     grouped so that consecutive workgroups of one XCD share a KV head.
#include "device_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int KT = 64;                 // keys per sub-tile
constexpr int kRelposLdsMax = 3073;    // table entries staged in LDS (2R+1 <= this)
constexpr float kRescaleThresh = 8.0f; // base-2 growth allowed before rescaling O

template <int D>
struct Lds {
  static constexpr int KROW = D * 2;          // bytes per K row
  static constexpr int VROW = KT * 2;         // bytes per V^T row (one head-dim index)
  static constexpr int KBYTES = KT * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int DOCBYTES = KT * 4;
  static constexpr int BUF = KBYTES + VBYTES + DOCBYTES;
};

// physical 16-byte chunk of K row `key`, logical chunk `ch`
__device__ __forceinline__ int k_off(int key, int ch, int krow) { return key * krow + ((ch ^ (key & 7)) << 4); }
// V^T row d, physical chunk pc (8 keys)
__device__ __forceinline__ int vt_off(int d, int pc) { return d * (KT * 2) + ((pc ^ (d & 7)) << 4); }

// key offset (within the 64-key sub-tile) held by S^T register rr of M-tile mt,
// excluding the lane-half term 4*half
__device__ __forceinline__ constexpr int key_of(int mt, int rr) { return 32 * mt + 8 * (rr >> 2) + (rr & 3); }

template <int D, int NW, int SCORE, int MK>
__global__ __launch_bounds__(NW * 64, 2) void prefill_kernel(FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;
  constexpr int DCH = D / 8;     // 16-byte chunks per row
  constexpr int KSTEPS = D / 16; // k-steps of the QK^T product
  constexpr int DM = D / 32;     // 32-row tiles of O^T
  constexpr int KCH = (KT * DCH + NT - 1) / NT;   // K chunks staged per thread
  constexpr int NQUAD = 16 * DCH;                 // V units of 4 keys x 8 dims
  constexpr int VQ = (NQUAD + NT - 1) / NT;
  constexpr bool kDoc = (MK == MK_INTERVAL_DOC);
  constexpr bool kRel = (SCORE == FA_S_RELPOS);
  using L = Lds<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::BUF];
  __shared__ float rel_lds[kRel ? kRelposLdsMax : 1];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // ---- work item: (b, h_q, r), longest rows first, heads grouped per XCD
  const int nbh = p.B * p.Hq;
  const int nqb = p.tab.nqb;
  const int Lid = blockIdx.x;
  int bh, r;
  if ((nbh & 7) == 0) {
    const int per = nbh >> 3, x = Lid & 7, jj = Lid >> 3;
    bh = x * per + jj % per;
    r = nqb - 1 - jj / per;
  } else {
    bh = Lid % nbh;
    r = nqb - 1 - Lid / nbh;
  }
  const int b = bh / p.Hq;
  const int hq = bh - b * p.Hq;
  const int hkv = hq / p.g;

  const int q_len = (int)p.q_len;
  const int kv_len = (int)p.kv_len;
  const int i_loc = r * BQ + w * 32 + col;
  const bool row_ok = i_loc < q_len;
  const int i_g = i_loc + (int)p.q_offset;
  const int i_wave0 = r * BQ + w * 32 + (int)p.q_offset;   // first row of the wave

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[row][16t + 8 half .. +8]
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qrow = p.q + ((int64_t)bh * p.q_len + (row_ok ? i_loc : 0)) * D;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4 v = row_ok ? load16(qrow + 16 * t + 8 * half) : u32x4{0, 0, 0, 0};
      qf[t] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- block-table row
  const int tb = p.tab.tB == 1 ? 0 : b;
  const int th = p.tab.tH == 1 ? 0 : hq;
  const int row = (tb * p.tab.tH + th) * nqb + r;
  const int nf = uniform(p.tab.fnum[row]);
  const int np = uniform(p.tab.num[row]);
  const int32_t* flist = p.tab.fidx + uniform(p.tab.fptr[row]);
  const int32_t* plist = p.tab.idx + uniform(p.tab.ptr[row]);
  const int spb = p.tab.bk / KT;
  const int nsub = (nf + np) * spb;

  const uint16_t* kbase = p.k + (int64_t)(b * p.Hkv + hkv) * p.kv_len * D;
  const uint16_t* vbase = p.v + (int64_t)(b * p.Hkv + hkv) * p.kv_len * D;
  const int32_t* docr = doc_row(p.doc, b);
  const int doc_i = (p.prog.has_doc && row_ok) ? docr[i_g] : 0;
  const ScoreCtx sc = make_score_ctx(p.score, p.scale, hq);

  // per-row allowed key interval of the pre-compiled mask (partial blocks only)
  uint32_t lo_u = 0, span = 0;
  if constexpr (MK != MK_GENERIC) {
    int lo = p.prog.wmin > 0 ? max(0, i_g - p.prog.wmin + 1) : 0;
    int hi = p.prog.hi_self ? i_g : (p.prog.pmin >= 0 ? max(p.prog.pmin - 1, i_g) : 0x7fffffff);
    hi = min(hi, kv_len - 1);
    if (hi >= lo) {
      lo_u = (uint32_t)lo;
      span = (uint32_t)(hi - lo);
    } else {
      lo_u = 0x80000000u;  // no key of any sub-tile can match
      span = 0;
    }
  }

  // relative-position table of this query head, pre-multiplied by log2(e)
  const int R = p.score.radius;
  const bool rel_in_lds = kRel && (2 * R + 1) <= kRelposLdsMax;
  if constexpr (kRel) {
    if (rel_in_lds) {
      for (int x = tid; x < 2 * R + 1; x += NT) rel_lds[x] = sc.tab[x] * kLog2e;
    }
  }

  auto sub_j0 = [&](int s, bool& partial) -> int {
    const int blk = s / spb;
    const int sub = s - blk * spb;
    partial = blk >= nf;
    const int c = partial ? plist[blk - nf] : flist[blk];
    return uniform(c) * p.tab.bk + sub * KT;
  };

  // ---- staging registers
  u32x4 kreg[KCH];
  u32x4 vreg[VQ][4];
  int dreg = 0;
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int f = tid + NT * u;
      const int key = f / DCH, ch = f % DCH;
      const int j = j0 + key;
      kreg[u] = (f < KT * DCH && (unsigned)j < (unsigned)kv_len) ? load16(kbase + (int64_t)j * D + ch * 8)
                                                                  : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VQ; ++u) {
      const int qd = tid + NT * u;
      const int kq = qd / DCH, dc = qd % DCH;
      const int tq = kq >> 2, a = (kq >> 1) & 1, hh = kq & 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 16 * tq + 8 * a + 4 * hh + e;
        vreg[u][e] = (qd < NQUAD && (unsigned)j < (unsigned)kv_len) ? load16(vbase + (int64_t)j * D + dc * 8)
                                                                    : u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (kDoc) {
      if (tid < KT) {
        const int j = j0 + tid;
        dreg = (unsigned)j < (unsigned)kv_len ? docr[j] : -1;
      }
    }
  };
  auto store_tile = [&](uint8_t* buf) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int f = tid + NT * u;
      if (f < KT * DCH) {
        const int key = f / DCH, ch = f % DCH;
        *reinterpret_cast<u32x4*>(buf + k_off(key, ch, L::KROW)) = kreg[u];
      }
    }
    uint8_t* vt = buf + L::KBYTES;
#pragma unroll
    for (int u = 0; u < VQ; ++u) {
      const int qd = tid + NT * u;
      if (qd < NQUAD) {
        const int kq = qd / DCH, dc = qd % DCH;
        const int tq = kq >> 2, a = (kq >> 1) & 1, hh = kq & 1;
#pragma unroll
        for (int dd = 0; dd < 8; dd += 2) {
          // two head-dim indices per source dword: low halves -> dd, high halves -> dd+1
          const uint32_t x0 = vreg[u][0][dd >> 1], x1 = vreg[u][1][dd >> 1];
          const uint32_t x2 = vreg[u][2][dd >> 1], x3 = vreg[u][3][dd >> 1];
          const u32x2 lo2 = {__builtin_amdgcn_perm(x1, x0, 0x05040100u), __builtin_amdgcn_perm(x3, x2, 0x05040100u)};
          const u32x2 hi2 = {__builtin_amdgcn_perm(x1, x0, 0x07060302u), __builtin_amdgcn_perm(x3, x2, 0x07060302u)};
          const int d = dc * 8 + dd;
          *reinterpret_cast<u32x2*>(vt + vt_off(d, 2 * tq + hh) + 8 * a) = lo2;
          *reinterpret_cast<u32x2*>(vt + vt_off(d + 1, 2 * tq + hh) + 8 * a) = hi2;
        }
      }
    }
    if constexpr (kDoc) {
      if (tid < KT) reinterpret_cast<int32_t*>(buf + L::KBYTES + L::VBYTES)[tid] = dreg;
    }
  };

  // ---- online softmax state (per lane: one query row; halves share m)
  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};

  bool part_cur = false;
  int j0_cur = 0;
  if (nsub > 0) {
    j0_cur = sub_j0(0, part_cur);
    load_tile(j0_cur);
  }

  for (int s = 0; s < nsub; ++s) {
    uint8_t* buf = smem + (s & 1) * L::BUF;
    store_tile(buf);
    __syncthreads();
    bool part_nxt = false;
    int j0_nxt = 0;
    if (s + 1 < nsub) {
      j0_nxt = sub_j0(s + 1, part_nxt);
      load_tile(j0_nxt);
    }

    // ---- S^T = K Q^T for the 64 keys of this sub-tile
    f32x16 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x16{};
      const int key = 32 * mt + col;
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(buf + k_off(key, 2 * t + half, L::KROW));
        sacc[mt] = mfma32(__builtin_bit_cast(bf16x8, kv), qf[t], sacc[mt]);
      }
    }

    const bool masked = part_cur || (j0_cur + KT > kv_len);
    const int jl = j0_cur + 4 * half;   // key of element (mt=0, rr=0) in this lane

    // ---- element mask (partial / ragged sub-tiles only): x = -inf where disallowed
    if (masked) {
      if constexpr (MK == MK_GENERIC) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int j = jl + key_of(mt, rr);
            bool ok = (unsigned)j < (unsigned)kv_len;
            if (part_cur && ok) ok = mask_allowed(p.prog, i_g, j, doc_i, p.prog.has_doc ? docr[j] : 0);
            sacc[mt][rr] = ok ? sacc[mt][rr] : kNegInf;
          }
      } else {
        const int32_t* dl = reinterpret_cast<const int32_t*>(buf + L::KBYTES + L::VBYTES);
        // keys outside [lo, hi] (hi already clipped to kv_len - 1) are masked; when only
        // the ragged tail needs masking the same interval test applies with the tail
        // bound alone
        uint32_t lo_t = lo_u, span_t = span;
        if (!part_cur) {
          lo_t = 0;
          span_t = (uint32_t)(kv_len - 1);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            int dq[4] = {doc_i, doc_i, doc_i, doc_i};
            if constexpr (kDoc) {
              if (part_cur) {
                const u32x4 dv = *reinterpret_cast<const u32x4*>(dl + 32 * mt + 8 * g4 + 4 * half);
                dq[0] = (int)dv[0];
                dq[1] = (int)dv[1];
                dq[2] = (int)dv[2];
                dq[3] = (int)dv[3];
              }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rr = 4 * g4 + e;
              const uint32_t j = (uint32_t)(jl + key_of(mt, rr));
              const bool ok = (j - lo_t) <= span_t && dq[e] == doc_i;
              sacc[mt][rr] = ok ? sacc[mt][rr] : kNegInf;
            }
          }
      }
    }

    // ---- score_mod to the base-2 domain and the tile maximum
    // Monotone kinds keep the raw score in sacc (tile maximum mapped once); the others
    // store t = log2(e) * score_mod(s * scale) in sacc.
    bool raw_mode;
    float bias2 = 0.f;  // constant base-2 bias of a saturated relative-position tile
    if constexpr (SCORE == FA_S_IDENTITY || SCORE == FA_S_SOFTCAP) {
      raw_mode = true;
    } else if constexpr (SCORE == FA_S_RELPOS) {
      const int dmin = i_wave0 - (j0_cur + KT - 1);
      const int dmax = i_wave0 + 31 - j0_cur;
      raw_mode = dmin >= R || dmax <= -R;
      if (raw_mode) bias2 = sc.tab[dmin >= R ? 2 * R : 0] * kLog2e;
    } else {
      raw_mode = false;
    }
    float tmax = kNegInf;
    if (raw_mode) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) tmax = fmaxf(tmax, sacc[mt][rr]);
    } else {
      if constexpr (SCORE == FA_S_ALIBI) {
        const float base = sc.slope2 * (float)(jl - i_g);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const float t = __builtin_fmaf(sacc[mt][rr], sc.c2, __builtin_fmaf(sc.slope2, (float)key_of(mt, rr), base));
            sacc[mt][rr] = t;
            tmax = fmaxf(tmax, t);
          }
      } else if constexpr (SCORE == FA_S_RELPOS) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            int rel = i_g - (jl + key_of(mt, rr));
            rel = rel < -R ? -R : (rel > R ? R : rel);
            const float bb = rel_in_lds ? rel_lds[rel + R] : sc.tab[rel + R] * kLog2e;
            const float t = __builtin_fmaf(sacc[mt][rr], sc.c2, bb);
            sacc[mt][rr] = t;
            tmax = fmaxf(tmax, t);
          }
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // map a raw-score maximum into the base-2 domain
    float m_cand = tmax;
    if (raw_mode && tmax != kNegInf) {
      if constexpr (SCORE == FA_S_SOFTCAP) {
        m_cand = sc.cap2 - 2.f * sc.cap2 * fast_rcp(fast_exp2(tmax * sc.capk) + 1.f);
      } else {
        m_cand = __builtin_fmaf(tmax, sc.c2, bias2);
      }
    }

    // ---- lazy online-softmax rescale (wave-uniform branch)
    const bool grow = m_cand > m_run + kRescaleThresh;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? m_cand : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;   // 0 when m_run = -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;

    // ---- weights P (bf16) and their row sum (fp32, before rounding)
    bf16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 pk;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float pv[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float x = sacc[t >> 1][8 * (t & 1) + 2 * e2 + h2];
          float arg;
          if constexpr (SCORE == FA_S_SOFTCAP) {
            const float rr = fast_rcp(fast_exp2(x * sc.capk) + 1.f);
            arg = __builtin_fmaf(-2.f * sc.cap2, rr, sc.cap2 - m_use);
            if (masked) arg = (x == kNegInf) ? kNegInf : arg;
          } else if constexpr (SCORE == FA_S_IDENTITY) {
            arg = __builtin_fmaf(x, sc.c2, -m_use);
          } else {
            arg = raw_mode ? __builtin_fmaf(x, sc.c2, bias2 - m_use) : x - m_use;
          }
          pv[h2] = fast_exp2(arg);
        }
        pk[e2] = pack_bf16x2(pv[0], pv[1]);
        psum += pv[0] + pv[1];
      }
      pb[t] = __builtin_bit_cast(bf16x8, pk);
    }
    l_run += psum;

    // ---- O^T += V^T P^T
    const uint8_t* vt = buf + L::KBYTES;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
      const int d = 32 * dm + col;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 vv = *reinterpret_cast<const u32x4*>(vt + vt_off(d, 2 * t + half));
        oacc[dm] = mfma32(__builtin_bit_cast(bf16x8, vv), pb[t], oacc[dm]);
      }
    }

    part_cur = part_nxt;
    j0_cur = j0_nxt;
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    uint16_t* orow = p.o + ((int64_t)bh * p.q_len + i_loc) * D;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dm + 8 * gq + 4 * half;
        u32x2 o2;
        o2[0] = pack_bf16x2(oacc[dm][4 * gq + 0] * inv, oacc[dm][4 * gq + 1] * inv);
        o2[1] = pack_bf16x2(oacc[dm][4 * gq + 2] * inv, oacc[dm][4 * gq + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = o2;
      }
    }
    if (half == 0) {
      p.lse[(int64_t)bh * p.q_len + i_loc] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <int D, int NW, int SCORE>
void launch_mk(const FwdParams& p, hipStream_t s, dim3 grid, dim3 block) {
  switch (p.prog.mk) {
    case MK_INTERVAL: hipLaunchKernelGGL((prefill_kernel<D, NW, SCORE, MK_INTERVAL>), grid, block, 0, s, p); break;
    case MK_INTERVAL_DOC: hipLaunchKernelGGL((prefill_kernel<D, NW, SCORE, MK_INTERVAL_DOC>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((prefill_kernel<D, NW, SCORE, MK_GENERIC>), grid, block, 0, s, p); break;
  }
}

template <int D, int NW>
hipError_t launch_nw(const FwdParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.Hq * p.tab.nqb));
  const dim3 block(NW * 64);
  switch (p.score.kind) {
    case FA_S_IDENTITY: launch_mk<D, NW, FA_S_IDENTITY>(p, s, grid, block); break;
    case FA_S_ALIBI: launch_mk<D, NW, FA_S_ALIBI>(p, s, grid, block); break;
    case FA_S_SOFTCAP: launch_mk<D, NW, FA_S_SOFTCAP>(p, s, grid, block); break;
    default: launch_mk<D, NW, FA_S_RELPOS>(p, s, grid, block); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const FwdParams& p, hipStream_t s) {
  if (p.B * p.Hq * p.tab.nqb == 0) return hipSuccess;
  const int nw = p.tab.bq / 32;
  if (p.d == 128) return nw == 4 ? launch_nw<128, 4>(p, s) : launch_nw<128, 2>(p, s);
  return nw == 4 ? launch_nw<64, 4>(p, s) : launch_nw<64, 2>(p, s);
}

}  // namespace fa
