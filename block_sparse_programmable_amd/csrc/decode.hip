// Split-KV decode for gfx950: short query (all rows in one query block), long KV.
//
// "FlexAttention: compiler optimization of custom attention", section 6 -- with one
// query per step the work is split along the KV length; each split produces a local
// (max, normaliser, unnormalised output) and the splits are merged with weights from
// their normalisers, an empty split contributing nothing.  "FlexAttention: from rules
// to fused kernels", section 3.2 (split-KV strict merge) -- the splits are balanced by
// the number of listed blocks, not by KV range, and averaging normalised split outputs
// would be wrong.  The merge law itself is "Kernels: turning logical sparsity into real
// speed", section 3.
//
// gfx950 mapping
//   * one workgroup (4 waves) per (b, h_kv, split); the g = Hq/Hkv query heads that share
//     a KV head, times q_len positions, form the 32 columns of one MFMA tile, so every
//     K/V byte is read from HBM once per (b, h_kv).
//   * a split is a contiguous range of the row's listed blocks with equal block counts.
//     Each iteration stages one 128-key block (K row-major, V transposed, both
//     XOR-swizzled) into LDS with 16-byte coalesced loads; the next block's loads are in
//     flight in registers while the current one is computed.  Wave w takes keys
//     32w .. 32w+31 of the block and keeps its own online-softmax state.
//   * the four wave states are merged through LDS at the end of the split and written
//     as (m, l, o) partials; a second small kernel merges the splits.
#include "device_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int DKT = 128;  // keys per decode iteration (one 128-key block)

template <int D>
struct DLds {
  static constexpr int KROW = D * 2;
  static constexpr int VROW = DKT * 2;
  static constexpr int KBYTES = DKT * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
};

__device__ __forceinline__ int dk_off(int key, int ch, int krow) { return key * krow + ((ch ^ (key & 7)) << 4); }
__device__ __forceinline__ int dvt_off(int d, int pc) { return d * (DKT * 2) + ((pc ^ (d & 7)) << 4); }

template <int D, int SCORE>
__global__ __launch_bounds__(256, 1) void decode_kernel(FwdParams p) {
  constexpr int NT = 256;
  constexpr int DCH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DM = D / 32;
  constexpr int KCH = DKT * DCH / NT;     // K chunks per thread
  constexpr int NQUAD = 32 * DCH;         // V units of 4 keys x 8 dims
  constexpr int VQ = NQUAD / NT;
  using L = DLds<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::BUF];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int ns = p.nsplit;
  const int s_id = blockIdx.x % ns;
  const int bk_id = blockIdx.x / ns;       // b * Hkv + h_kv
  const int b = bk_id / p.Hkv;
  const int hkv = bk_id - b * p.Hkv;
  const int q_len = (int)p.q_len;
  const int kv_len = (int)p.kv_len;

  // column -> (query head, position)
  const int ncols = p.g * q_len;
  const bool col_ok = col < ncols;
  const int hh = col_ok ? col / q_len : 0;
  const int ip = col_ok ? col - hh * q_len : 0;
  const int hq = hkv * p.g + hh;
  const int i_g = ip + (int)p.q_offset;
  const int64_t orow = ((int64_t)(b * p.Hq + hq)) * p.q_len + ip;

  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qrow = p.q + orow * D;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4 v = col_ok ? load16(qrow + 16 * t + 8 * half) : u32x4{0, 0, 0, 0};
      qf[t] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // block-table row shared by the query heads of this KV head
  const int tb = p.tab.tB == 1 ? 0 : b;
  const int th = p.tab.tH == 1 ? 0 : hkv * p.g;
  const int row = (tb * p.tab.tH + th) * p.tab.nqb;
  const int nf = uniform(p.tab.fnum[row]);
  const int np = uniform(p.tab.num[row]);
  const int32_t* flist = p.tab.fidx + uniform(p.tab.fptr[row]);
  const int32_t* plist = p.tab.idx + uniform(p.tab.ptr[row]);
  const int n_ent = nf + np;
  const int e_begin = (int)(((int64_t)s_id * n_ent) / ns);
  const int e_end = (int)(((int64_t)(s_id + 1) * n_ent) / ns);

  const uint16_t* kbase = p.k + (int64_t)bk_id * p.kv_len * D;
  const uint16_t* vbase = p.v + (int64_t)bk_id * p.kv_len * D;
  const int32_t* docr = doc_row(p.doc, b);
  const int doc_i = (p.prog.has_doc && col_ok) ? docr[i_g] : 0;
  const ScoreCtx sc = make_score_ctx(p.score, p.scale, hq);

  auto ent_j0 = [&](int e, bool& partial) -> int {
    partial = e >= nf;
    const int c = partial ? plist[e - nf] : flist[e];
    return uniform(c) * DKT;
  };

  u32x4 kreg[KCH];
  u32x4 vreg[VQ][4];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int f = tid + NT * u;
      const int key = f / DCH, ch = f % DCH;
      const int j = j0 + key;
      kreg[u] = (unsigned)j < (unsigned)kv_len ? load16(kbase + (int64_t)j * D + ch * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VQ; ++u) {
      const int qd = tid + NT * u;
      const int kq = qd / DCH, dc = qd % DCH;
      const int ww = kq >> 3, tq = (kq >> 2) & 1, a = (kq >> 1) & 1, h2 = kq & 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 32 * ww + 16 * tq + 8 * a + 4 * h2 + e;
        vreg[u][e] = (unsigned)j < (unsigned)kv_len ? load16(vbase + (int64_t)j * D + dc * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](uint8_t* buf) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int f = tid + NT * u;
      const int key = f / DCH, ch = f % DCH;
      *reinterpret_cast<u32x4*>(buf + dk_off(key, ch, L::KROW)) = kreg[u];
    }
    uint8_t* vt = buf + L::KBYTES;
#pragma unroll
    for (int u = 0; u < VQ; ++u) {
      const int qd = tid + NT * u;
      const int kq = qd / DCH, dc = qd % DCH;
      const int ww = kq >> 3, tq = (kq >> 2) & 1, a = (kq >> 1) & 1, h2 = kq & 1;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int sh = (dd & 1) * 16;
        const uint32_t e0 = (vreg[u][0][dd >> 1] >> sh) & 0xffffu;
        const uint32_t e1 = (vreg[u][1][dd >> 1] >> sh) & 0xffffu;
        const uint32_t e2 = (vreg[u][2][dd >> 1] >> sh) & 0xffffu;
        const uint32_t e3 = (vreg[u][3][dd >> 1] >> sh) & 0xffffu;
        const int d = dc * 8 + dd;
        *reinterpret_cast<u32x2*>(vt + dvt_off(d, 4 * ww + 2 * tq + h2) + 8 * a) =
            u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
      }
    }
  };

  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};

  bool part_cur = false;
  int j0_cur = 0;
  if (e_begin < e_end) {
    j0_cur = ent_j0(e_begin, part_cur);
    load_tile(j0_cur);
  }
  for (int e = e_begin; e < e_end; ++e) {
    uint8_t* buf = smem + ((e - e_begin) & 1) * L::BUF;
    store_tile(buf);
    __syncthreads();
    bool part_nxt = false;
    int j0_nxt = 0;
    if (e + 1 < e_end) {
      j0_nxt = ent_j0(e + 1, part_nxt);
      load_tile(j0_nxt);
    }

    // S^T for keys 32w .. 32w+31 of the block
    f32x16 sacc = f32x16{};
    const int key = 32 * w + col;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(buf + dk_off(key, 2 * t + half, L::KROW));
      sacc = mfma32(__builtin_bit_cast(bf16x8, kv), qf[t], sacc);
    }

    const bool ragged = j0_cur + DKT > kv_len;
    float tmax = kNegInf;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int j = j0_cur + 32 * w + 8 * (rr >> 2) + 4 * half + (rr & 3);
      float t = score_log2<SCORE>(sacc[rr], sc, i_g, j);
      if (ragged || part_cur) {
        bool ok = (unsigned)j < (unsigned)kv_len;
        if (part_cur && ok) {
          const int doc_j = p.prog.has_doc ? docr[j] : 0;
          ok = mask_allowed(p.prog, i_g, j, doc_i, doc_j);
        }
        t = ok ? t : kNegInf;
      }
      sacc[rr] = t;
      tmax = fmaxf(tmax, t);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;

    bf16x8 pb[2];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 pk;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float p0 = fast_exp2(sacc[8 * t + 2 * e2] - m_use);
        const float p1 = fast_exp2(sacc[8 * t + 2 * e2 + 1] - m_use);
        psum += p0 + p1;
        pk[e2] = pack_bf16x2(p0, p1);
      }
      pb[t] = __builtin_bit_cast(bf16x8, pk);
    }
    l_run += psum;

    const uint8_t* vt = buf + L::KBYTES;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
      const int d = 32 * dm + col;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 vv = *reinterpret_cast<const u32x4*>(vt + dvt_off(d, 4 * w + 2 * t + half));
        oacc[dm] = mfma32(__builtin_bit_cast(bf16x8, vv), pb[t], oacc[dm]);
      }
    }
    part_cur = part_nxt;
    j0_cur = j0_nxt;
  }

  // ---- merge the four wave states through LDS, write this split's partial
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);            // [4][32] m, [4][32] l, [4][D][32] o
  float* red_m = red;
  float* red_l = red + 4 * 32;
  float* red_o = red + 8 * 32;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (half == 0) {
    red_m[w * 32 + col] = m_run;
    red_l[w * 32 + col] = l_tot;
  }
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int d = 32 * dm + 8 * (rr >> 2) + 4 * half + (rr & 3);
      red_o[(w * D + d) * 32 + col] = oacc[dm][rr];
    }
  }
  __syncthreads();
  // thread t: column c = t % 32, dims (t / 32) + 8k
  {
    const int c = tid & 31;
    if (c < ncols) {
      float M = kNegInf;
#pragma unroll
      for (int q = 0; q < 4; ++q) M = fmaxf(M, red_m[q * 32 + c]);
      float wq[4];
      float lsum = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float mq = red_m[q * 32 + c];
        wq[q] = (mq == kNegInf) ? 0.f : fast_exp2(mq - M);
        lsum += wq[q] * red_l[q * 32 + c];
      }
      const int hh2 = c / q_len;
      const int ip2 = c - hh2 * q_len;
      const int64_t prow = (((int64_t)(b * p.Hq + hkv * p.g + hh2)) * p.q_len + ip2) * ns + s_id;
      float* ws_m = p.ws;
      float* ws_l = p.ws + (int64_t)p.B * p.Hq * p.q_len * ns;
      float* ws_o = p.ws + 2 * (int64_t)p.B * p.Hq * p.q_len * ns;
      if ((tid >> 5) == 0) {
        ws_m[prow] = M;
        ws_l[prow] = lsum;
      }
      for (int d = tid >> 5; d < D; d += 8) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc += wq[q] * red_o[(q * D + d) * 32 + c];
        ws_o[prow * D + d] = acc;
      }
    }
  }
}

// one wave per output row: merge the split partials (base-2 maxima)
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(FwdParams p) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.q_len;
  const int64_t rowi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rowi >= rows) return;
  const int ns = p.nsplit;
  const float* ws_m = p.ws;
  const float* ws_l = p.ws + rows * ns;
  const float* ws_o = p.ws + 2 * rows * ns;
  float M = kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ws_m[rowi * ns + s]);
  float lsum = 0.f;
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ms = ws_m[rowi * ns + s];
    const float wgt = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
    lsum += wgt * ws_l[rowi * ns + s];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] += wgt * ws_o[(rowi * ns + s) * D + lane * PER + k];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* o = p.o + rowi * D + lane * PER;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    const uint32_t pk = pack_bf16x2(acc[0] * inv, 0.f);
    o[0] = (uint16_t)(pk & 0xffffu);
  }
  if (lane == 0) p.lse[rowi] = lsum > 0.f ? (M + fast_log2(lsum)) * kLn2 : kNegInf;
}

}  // namespace

bool decode_eligible(const FwdParams& p) {
  return p.tab.nqb == 1 && p.tab.bk == DKT && (int64_t)p.g * p.q_len <= 32 && p.q_len >= 1;
}

int32_t decode_splits(const FwdParams& p, int num_cus) {
  const int64_t items = (int64_t)p.B * p.Hkv;
  int64_t ns = (4 * (int64_t)num_cus + items - 1) / items;
  if (ns > p.tab.nkb) ns = p.tab.nkb;
  if (ns > 64) ns = 64;
  if (ns < 1) ns = 1;
  return (int32_t)ns;
}

size_t decode_workspace_bytes(const FwdParams& p, int32_t nsplit) {
  const size_t rows = (size_t)p.B * p.Hq * p.q_len;
  return rows * nsplit * (2 + (size_t)p.d) * sizeof(float);
}

hipError_t launch_decode(const FwdParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * p.nsplit));
  const dim3 block(256);
#define FA_DEC(DD, SS) hipLaunchKernelGGL((decode_kernel<DD, SS>), grid, block, 0, s, p)
  if (p.d == 128) {
    switch (p.score.kind) {
      case FA_S_IDENTITY: FA_DEC(128, FA_S_IDENTITY); break;
      case FA_S_ALIBI: FA_DEC(128, FA_S_ALIBI); break;
      case FA_S_SOFTCAP: FA_DEC(128, FA_S_SOFTCAP); break;
      default: FA_DEC(128, FA_S_RELPOS); break;
    }
  } else {
    switch (p.score.kind) {
      case FA_S_IDENTITY: FA_DEC(64, FA_S_IDENTITY); break;
      case FA_S_ALIBI: FA_DEC(64, FA_S_ALIBI); break;
      case FA_S_SOFTCAP: FA_DEC(64, FA_S_SOFTCAP); break;
      default: FA_DEC(64, FA_S_RELPOS); break;
    }
  }
#undef FA_DEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.B * p.Hq * p.q_len;
  const dim3 cgrid((unsigned)((rows + 3) / 4));
  if (p.d == 128) hipLaunchKernelGGL((combine_kernel<128>), cgrid, block, 0, s, p);
  else hipLaunchKernelGGL((combine_kernel<64>), cgrid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
