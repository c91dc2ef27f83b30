// Block-sparse attention forward, prefill shape (many query rows), for gfx950.
//
// One workgroup owns one query block (b, h_q, r) and walks the KV blocks that the
// block table lists for its row: first the FULL list, then the PARTIAL list
// ("FlexAttention: compiler optimization of custom attention", section 3 -- the
// forward fixes a query tile, reads the KV block numbers from the BlockMask and, for
// each kept block, computes Q K^T * scale, applies score_mod, applies mask_mod only
// on partial blocks, then updates the online softmax and accumulates with V).
// Online softmax state and merge law: "Kernels: turning logical sparsity into real
// speed", section 3; "Flash Attention self-test answers", Q24-Q29.
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
//   * softmax runs in base 2 with scale*log2(e) folded into one multiply.
//   * grid order: longest rows first (query block index descending), and heads
//     grouped so that consecutive workgroups of one XCD share a KV head.
#include "device_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int KT = 64;  // keys per sub-tile

template <int D>
struct Lds {
  static constexpr int KROW = D * 2;          // bytes per K row
  static constexpr int VROW = KT * 2;         // bytes per V^T row (one head-dim index)
  static constexpr int KBYTES = KT * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
};

// physical 16-byte chunk of K row `key`, logical chunk `ch`
__device__ __forceinline__ int k_off(int key, int ch, int krow) { return key * krow + ((ch ^ (key & 7)) << 4); }
// V^T row d, physical chunk pc (8 keys)
__device__ __forceinline__ int vt_off(int d, int pc) { return d * (KT * 2) + ((pc ^ (d & 7)) << 4); }

template <int D, int NW, int SCORE>
__global__ __launch_bounds__(NW * 64, 2) void prefill_kernel(FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;
  constexpr int DCH = D / 8;     // 16-byte chunks per row
  constexpr int KSTEPS = D / 16; // k-steps of the QK^T product
  constexpr int DM = D / 32;     // 32-row tiles of O^T
  constexpr int KCH = (KT * DCH + NT - 1) / NT;   // K chunks staged per thread
  constexpr int NQUAD = 16 * DCH;                 // V units of 4 keys x 8 dims
  constexpr int VQ = (NQUAD + NT - 1) / NT;
  using L = Lds<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::BUF];

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
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int f = tid + NT * u;
      const int key = f / DCH, ch = f % DCH;
      const int j = j0 + key;
      kreg[u] = (f < KT * DCH && (unsigned)j < (unsigned)kv_len) ? load16(kbase + (int64_t)j * D + ch * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VQ; ++u) {
      const int qd = tid + NT * u;
      const int kq = qd / DCH, dc = qd % DCH;
      const int tq = kq >> 2, a = (kq >> 1) & 1, hh = kq & 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 16 * tq + 8 * a + 4 * hh + e;
        vreg[u][e] = (qd < NQUAD && (unsigned)j < (unsigned)kv_len) ? load16(vbase + (int64_t)j * D + dc * 8) : u32x4{0, 0, 0, 0};
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
        for (int dd = 0; dd < 8; ++dd) {
          const int sh = (dd & 1) * 16;
          const uint32_t e0 = (vreg[u][0][dd >> 1] >> sh) & 0xffffu;
          const uint32_t e1 = (vreg[u][1][dd >> 1] >> sh) & 0xffffu;
          const uint32_t e2 = (vreg[u][2][dd >> 1] >> sh) & 0xffffu;
          const uint32_t e3 = (vreg[u][3][dd >> 1] >> sh) & 0xffffu;
          const int d = dc * 8 + dd;
          *reinterpret_cast<u32x2*>(vt + vt_off(d, 2 * tq + hh) + 8 * a) = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
        }
      }
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

    // ---- score_mod (log2 domain) and mask on partial / ragged sub-tiles
    const bool ragged = j0_cur + KT > kv_len;
    float tmax = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int j = j0_cur + 32 * mt + 8 * (rr >> 2) + 4 * half + (rr & 3);
        float t = score_log2<SCORE>(sacc[mt][rr], sc, i_g, j);
        if (ragged || part_cur) {
          bool ok = (unsigned)j < (unsigned)kv_len;
          if (part_cur && ok) {
            const int doc_j = p.prog.has_doc ? docr[j] : 0;
            ok = mask_allowed(p.prog, i_g, j, doc_i, doc_j);
          }
          t = ok ? t : kNegInf;
        }
        sacc[mt][rr] = t;
        tmax = fmaxf(tmax, t);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));

    // ---- online softmax update
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;

    bf16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 pk;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float p0 = fast_exp2(sacc[t >> 1][8 * (t & 1) + 2 * e2] - m_use);
        const float p1 = fast_exp2(sacc[t >> 1][8 * (t & 1) + 2 * e2 + 1] - m_use);
        psum += p0 + p1;
        pk[e2] = pack_bf16x2(p0, p1);
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

template <int D, int NW>
hipError_t launch_nw(const FwdParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.Hq * p.tab.nqb));
  const dim3 block(NW * 64);
  switch (p.score.kind) {
    case FA_S_IDENTITY: hipLaunchKernelGGL((prefill_kernel<D, NW, FA_S_IDENTITY>), grid, block, 0, s, p); break;
    case FA_S_ALIBI: hipLaunchKernelGGL((prefill_kernel<D, NW, FA_S_ALIBI>), grid, block, 0, s, p); break;
    case FA_S_SOFTCAP: hipLaunchKernelGGL((prefill_kernel<D, NW, FA_S_SOFTCAP>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((prefill_kernel<D, NW, FA_S_RELPOS>), grid, block, 0, s, p); break;
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
