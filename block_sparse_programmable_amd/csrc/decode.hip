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
// gfx950 mapping (the kernel is bound by HBM bandwidth, so the design maximises the
// bytes in flight per CU):
//   * a work unit is (b, h_kv, split); the g = Hq/Hkv query heads that share the KV head,
//     times q_len positions, form the columns of one 32-column MFMA tile, so every K/V
//     byte is read from HBM once per (b, h_kv).  A split is a contiguous range of the
//     row's listed blocks with equal block counts.
//   * each wave runs one unit on its own: no barriers.  It streams 32-key stages
//     HBM -> LDS with global_load_lds_dwordx4 (no staging registers) into a private ring
//     of kStages slots and keeps kStages - 1 stages in flight while it computes one;
//     a vmcnt wait per stage is the only synchronisation.  The ring of two waves fills
//     most of the LDS, so up to ~96 KB per CU are in flight.
//   * K and V of a stage are row-major in LDS with the XOR swizzles of the prefill
//     kernels (K 16-byte chunks by key & 7, V 32-byte units by key & 7): scores from
//     ds_read_b128 fragments, the P V operand from ds_read_b64_tr_b16.
//   * with one split the wave writes O and LSE itself; otherwise it writes its
//     (m, l, o) partial and a second small kernel merges the splits.
#include "device_common.hpp"
#include "fa_internal.hpp"
#include "prefill_common.hpp"

namespace fa {

namespace {

constexpr int DKT = 128;     // block size of the block table rows decoded here
constexpr int SK = 32;       // keys per stage
constexpr int kStages = 4;   // LDS ring slots per wave
constexpr int kDecWaves = 2; // independent waves (units) per workgroup

template <int D>
struct DLds {
  static constexpr int KROW = D * 2;            // bytes per K or V row
  static constexpr int HALF = SK * KROW;        // K (or V) part of a stage
  static constexpr int STAGE = 2 * HALF;        // K then V
  static constexpr int WAVE = kStages * STAGE;  // one wave's ring
  static constexpr int UNITS = D / 16;          // 32-byte units per V row
};

template <int D, int SCORE>
__global__ __launch_bounds__(64 * kDecWaves, 1) void decode_kernel(FwdParams p) {
  constexpr int DCH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DM = D / 32;
  constexpr int KPK = 1024 / (D * 2);          // keys per 1 KB copy
  constexpr int CPO = SK / KPK;                // copies per operand per stage
  constexpr int CPS = 2 * CPO;                 // copies per stage
  constexpr int VAR = KPK >= 8 ? 1 : 8 / KPK;
  using L = DLds<D>;
  static_assert(CPS * (kStages - 1) <= 63, "outstanding copies must fit the vmcnt counter");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDecWaves * L::WAVE];

  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int ns = p.nsplit;
  const int64_t unit = (int64_t)blockIdx.x * kDecWaves + w;
  const int64_t units = (int64_t)p.B * p.Hkv * ns;
  if (unit >= units) return;   // wave-uniform: no barrier follows
  const int s_id = (int)(unit % ns);
  const int bk_id = (int)(unit / ns);      // b * Hkv + h_kv
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
  const int nst = (e_end - e_begin) * (DKT / SK);

  const uint16_t* kbase = p.k + (int64_t)bk_id * p.kv_len * D;
  const uint16_t* vbase = p.v + (int64_t)bk_id * p.kv_len * D;
  const int32_t* docr = doc_row(p.doc, b);
  const int doc_i = (p.prog.has_doc && col_ok) ? docr[i_g] : 0;
  const ScoreCtx sc = make_score_ctx(p.score, p.scale, hq);

  // the unit's block list, 64 entries per register (lane e holds entry base + e)
  int lst_base = 0;
  auto load_list = [&](int base) -> int {
    const int e = e_begin + base + lane;
    return e < e_end ? (e < nf ? flist[e] : plist[e - nf]) : 0;
  };
  int lst = load_list(0);
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) asm volatile("" : "+v"(qf[t]));
  asm volatile("" : "+v"(lst));   // loads complete before the copies start
  auto stage_j0 = [&](int s) -> int {
    const int e = s / (DKT / SK);
    if (e - lst_base >= 64) {   // rare: next 64 entries (waits for all copies in flight)
      lst_base += 64;
      lst = load_list(lst_base);
    }
    return __builtin_amdgcn_readlane(lst, e - lst_base) * DKT + (s % (DKT / SK)) * SK;
  };
  auto stage_part = [&](int s) -> bool { return e_begin + s / (DKT / SK) >= nf; };

  // per-lane copy offsets (swizzles as in the prefill kernels)
  uint32_t koff[VAR], voff[VAR];
#pragma unroll
  for (int var = 0; var < VAR; ++var) {
    const int key_in = lane / DCH;
    const int pc = lane % DCH;
    const int key7 = (var * KPK + key_in) & 7;
    koff[var] = (uint32_t)(key_in * L::KROW + ((pc ^ key7) << 4));
    voff[var] = (uint32_t)(key_in * L::KROW + ((2 * (((pc >> 1) ^ key7) & (L::UNITS - 1)) + (pc & 1)) << 4));
  }
  uint8_t* ring = smem + w * L::WAVE;
  const uint32_t ring_lds = lds_addr(ring);

  // one stage (32 keys from j0) into ring slot `slot`
  auto copy_stage = [&](int j0, int slot) {
    const uint32_t mk = sreg(ring_lds + (uint32_t)slot * L::STAGE);
    const uint32_t mv = mk + L::HALF;
    if (j0 + SK <= kv_len) {
      const char* kg = (const char*)kbase + (int64_t)j0 * L::KROW;
      const char* vg = (const char*)vbase + (int64_t)j0 * L::KROW;
      static_for<CPO>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int grp = (u / 4) * 4096;   // immediate offsets stay below 4 KB
        dma16_s<(u % 4) * 1024>(mk + grp, kg + grp, koff[u % VAR]);
        dma16_s<(u % 4) * 1024>(mv + grp, vg + grp, voff[u % VAR]);
      });
    } else {
      // ragged tail: keys past kv_len re-read the last key (they are masked); offsets
      // from jb = min(j0, kv_len - 1) stay non-negative
      const int jb = min(j0, kv_len - 1);
      const char* kg = (const char*)kbase + (int64_t)jb * L::KROW;
      const char* vg = (const char*)vbase + (int64_t)jb * L::KROW;
      static_for<CPO>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const int key = u * KPK + lane / DCH;
        const uint32_t rowoff = (uint32_t)(min(j0 + key, kv_len - 1) - jb) * L::KROW;
        dma16_s<0>(mk + u * 1024, kg, rowoff + (koff[u % VAR] & (L::KROW - 1)));
        dma16_s<0>(mv + u * 1024, vg, rowoff + (voff[u % VAR] & (L::KROW - 1)));
      });
    }
  };

  // per-lane LDS read bases: K fragment t (key col, chunk 2t + half), V^T fragment of
  // head-dim tile dm (keys 4 half + (li >> 2) (+8, +16 per k-step), d0 = 32 dm + ...)
  const int g16 = lane >> 4, li = lane & 15;
  uint32_t kaddr[4], vaddr[DM];
#pragma unroll
  for (int t = 0; t < 4; ++t) kaddr[t] = (uint32_t)k_off(col, 2 * t + half, L::KROW);
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
    vaddr[dm] = (uint32_t)v_off<D>(4 * half + (li >> 2), 32 * dm + 16 * (g16 & 1) + 4 * (li & 3));

  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};

  // prologue: fill the ring
  int issued = 0;
  int j0_of[kStages];
#pragma unroll
  for (int k = 0; k < kStages; ++k) {
    if (k < nst) {
      j0_of[k] = stage_j0(k);
      copy_stage(j0_of[k], k);
      ++issued;
    }
  }

  for (int s = 0; s < nst; ++s) {
    const int slot = s % kStages;
    // stage s has landed once at most (issued - s - 1) stages of copies are outstanding
    switch (issued - s - 1) {
      case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(%0)" :: "i"(CPS) : "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(%0)" :: "i"(2 * CPS) : "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(%0)" :: "i"(3 * CPS) : "memory"); break;
    }
    int j0 = 0;
#pragma unroll
    for (int k = 0; k < kStages; ++k)
      if (k == slot) j0 = j0_of[k];
    const bool part = stage_part(s);
    const uint8_t* kb = ring + slot * L::STAGE;
    const uint8_t* vb = kb + L::HALF;

    // S^T for the 32 keys of the stage
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kb + kaddr[t & 3] + (t >> 2) * 128);
      sacc = mfma32(__builtin_bit_cast(bf16x8, kv), qf[t], sacc);
    }

    // score_mod first, then the mask (-inf) on partial and ragged stages only
    const int jl = j0 + 4 * half;   // key of register 0 in this lane
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sacc[rr] = score_log2<SCORE>(sacc[rr], sc, i_g, jl + key_of(0, rr));
    if (part || j0 + SK > kv_len) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int j = jl + key_of(0, rr);
        bool ok = (unsigned)j < (unsigned)kv_len;
        if (part && ok) ok = mask_allowed(p.prog, i_g, j, doc_i, p.prog.has_doc ? docr[j] : 0);
        sacc[rr] = ok ? sacc[rr] : kNegInf;
      }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) tmax = fmaxf(tmax, sacc[rr]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    if (m_new > m_run) {
      const float alpha = fast_exp2(m_run - m_use);   // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
    }
    m_run = m_new;

    float psum = 0.f;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      u32x4 pk;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float p0 = fast_exp2(sacc[8 * t2 + 2 * e2] - m_use);
        const float p1 = fast_exp2(sacc[8 * t2 + 2 * e2 + 1] - m_use);
        psum += p0 + p1;
        pk[e2] = cvt_pk_bf16(p0, p1);
      }
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const uint8_t* va = vb + vaddr[dm] + 16 * t2 * L::KROW;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(va));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(va + 8 * L::KROW));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[dm] = mfma32(a, pb, oacc[dm]);
      }
    }
    l_run += psum;

    // refill this slot with stage s + kStages once its reads have completed
    if (s + kStages < nst) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int jn = stage_j0(s + kStages);
#pragma unroll
      for (int k = 0; k < kStages; ++k)
        if (k == slot) j0_of[k] = jn;
      copy_stage(jn, slot);
      ++issued;
    }
  }

  // ---- results: final O and LSE (one split) or this split's (m, l, o) partial
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!col_ok) return;
  if (ns == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* o = p.o + orow * D;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dm + 8 * gq + 4 * half;
        u32x2 o2;
        o2[0] = cvt_pk_bf16(oacc[dm][4 * gq + 0] * inv, oacc[dm][4 * gq + 1] * inv);
        o2[1] = cvt_pk_bf16(oacc[dm][4 * gq + 2] * inv, oacc[dm][4 * gq + 3] * inv);
        *reinterpret_cast<u32x2*>(o + d0) = o2;
      }
    }
    if (half == 0) p.lse[orow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  } else {
    const int64_t rows = (int64_t)p.B * p.Hq * p.q_len;
    const int64_t prow = orow * ns + s_id;
    float* ws_m = p.ws;
    float* ws_l = p.ws + rows * ns;
    float* ws_o = p.ws + 2 * rows * ns;
    if (half == 0) {
      ws_m[prow] = m_run;
      ws_l[prow] = l_tot;
    }
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dm + 8 * gq + 4 * half;
        f32x4 v4 = {oacc[dm][4 * gq + 0], oacc[dm][4 * gq + 1], oacc[dm][4 * gq + 2], oacc[dm][4 * gq + 3]};
        *reinterpret_cast<f32x4*>(ws_o + prow * D + d0) = v4;
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
    *reinterpret_cast<uint32_t*>(o) = cvt_pk_bf16(acc[0] * inv, acc[1] * inv);
  } else {
    const uint32_t pk = cvt_pk_bf16(acc[0] * inv, 0.f);
    o[0] = (uint16_t)(pk & 0xffffu);
  }
  if (lane == 0) p.lse[rowi] = lsum > 0.f ? (M + fast_log2(lsum)) * kLn2 : kNegInf;
}

}  // namespace

bool decode_eligible(const FwdParams& p) {
  return p.tab.nqb == 1 && p.tab.bk == DKT && (int64_t)p.g * p.q_len <= 32 && p.q_len >= 1;
}

// splits per (b, h_kv): enough units for one wave per SIMD pair slot (kDecWaves waves per
// CU, one workgroup per CU), capped by the listed block count of a row
int32_t decode_splits(const FwdParams& p, int num_cus) {
  const int64_t items = (int64_t)p.B * p.Hkv;
  const int64_t slots = (int64_t)kDecWaves * num_cus;
  int64_t ns = (slots + items - 1) / items;
  if (ns > p.tab.nkb) ns = p.tab.nkb;
  if (ns > 64) ns = 64;
  if (ns < 1) ns = 1;
  return (int32_t)ns;
}

size_t decode_workspace_bytes(const FwdParams& p, int32_t nsplit) {
  if (nsplit <= 1) return 0;   // one split writes O and LSE directly
  const size_t rows = (size_t)p.B * p.Hq * p.q_len;
  return rows * nsplit * (2 + (size_t)p.d) * sizeof(float);
}

hipError_t launch_decode(const FwdParams& p, hipStream_t s) {
  const int64_t units = (int64_t)p.B * p.Hkv * p.nsplit;
  const dim3 grid((unsigned)((units + kDecWaves - 1) / kDecWaves));
  const dim3 block(64 * kDecWaves);
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
  if (e != hipSuccess || p.nsplit <= 1) return e;
  const int64_t rows = (int64_t)p.B * p.Hq * p.q_len;
  const dim3 cgrid((unsigned)((rows + 3) / 4));
  if (p.d == 128) hipLaunchKernelGGL((combine_kernel<128>), cgrid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((combine_kernel<64>), cgrid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
