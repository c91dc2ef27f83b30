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
// gfx950 mapping (the kernel is bound by HBM bandwidth, so the design keeps many bytes
// in flight per CU and little work per byte):
//   * a work unit is (b, h_kv, split); the g = Hq/Hkv query heads that share the KV head,
//     times q_len positions (at most 16), form the columns of 16x16x32 MFMA tiles, so
//     every K/V byte is read from HBM once per (b, h_kv).  A split is a contiguous range
//     of the row's listed blocks with equal block counts.
//   * each wave runs one unit on its own: no barriers.  It streams 16-key stages
//     HBM -> LDS with global_load_lds_dwordx4 (no staging registers) into a private
//     ring of NS slots and keeps NS - 1 stages in flight while it computes one; a vmcnt
//     wait per stage is the only synchronisation.  A slot holds the stage's K rows,
//     then its V rows, then (position-table score_mod only) the 1 KB of table entries
//     of its 16 columns x 16 keys.  NS = 5 (8 KB slots at d = 128, 160 KB for the four
//     waves of a workgroup) for every score_mod but the position table, whose larger
//     slots leave room for NS = 4 (144 KB at d = 128).
//   * K and V of a stage are row-major in LDS with the XOR swizzles of the prefill
//     kernels (conflict-free on the 64-bank LDS): scores from ds_read_b128 fragments,
//     the P V operand from ds_read_b64_tr_b16.
//   * with one split the wave writes O and LSE itself; when the splits of a (b, h_kv)
//     share a workgroup they are merged through LDS after the stream; otherwise each
//     wave writes its (m, l, o) partial and a second small kernel merges the splits.
#include "device_common.hpp"
#include "fa_internal.hpp"
#include "prefill_common.hpp"

namespace fa {

namespace {

constexpr int DKT = 128;     // block size of the block table rows decoded here
constexpr int SK = 16;       // keys per stage
constexpr int kStages = 5;   // LDS ring slots per wave
constexpr int kDecWaves = 4; // independent waves (units) per workgroup
constexpr int kDecCols = 16; // query columns (heads sharing a KV head x positions)

template <int D, int NS, int XW>
struct DLds {
  static constexpr int KROW = D * 2;            // bytes per K or V row
  static constexpr int HALF = SK * KROW;        // K (or V) part of a stage
  static constexpr int STAGE = 2 * HALF + XW;   // K, V, then XW bytes of table window
  static constexpr int WAVE = NS * STAGE;       // one wave's ring of NS slots
  static constexpr int UNITS = D / 16;          // 32-byte units per V row
};

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  // D[i][n] += sum_k A[i][k] B[k][n]; lane l holds A[l%16][8(l/16)..+8] and
  // B[8(l/16)..+8][l%16]; D: lane l, register r -> row 4(l/16) + r, column l%16.
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k16(const s16x4& a, const s16x4& b, const f32x4& c) {
  // as above with a 16-deep contraction: lane l holds A[l%16][4(l/16)..+4] and
  // B[4(l/16)..+4][l%16]
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Scores S^T (keys x columns) of a 16-key stage on 16x16x32 MFMAs (contraction over the
// head dim), O^T (head-dim x columns) on 16x16x16 MFMAs (contraction over the stage's
// keys).  In lane l (group g = l/16, column l%16) S^T register r holds key 4g + r,
// which is exactly the P^T operand of the P V product; the V^T operand of lane l
// (d = 16 dt + l%16, keys 4g .. 4g+3) is one transposing LDS read.
template <int D, int SCORE, bool PAGED>
__global__ __launch_bounds__(64 * kDecWaves, 1) void decode_kernel(FwdParams p) {
  constexpr int DCH = D / 8;
  constexpr int KT4 = D / 32;                  // k-steps of the QK product
  constexpr int DT = D / 16;                   // 16-row tiles of O^T
  constexpr int KPK = 1024 / (D * 2);          // keys per 1 KB copy
  constexpr int CPO = SK / KPK;                // copies per operand per stage
  constexpr int CPS = 2 * CPO;                 // copies per stage
  constexpr int KVAR = KPK >= kSwzKeys ? 1 : kSwzKeys / KPK;   // K swizzle patterns per stage
  constexpr int VVAR = KPK >= 8 ? 1 : 8 / KPK;                  // V pattern repeats every 8 keys
  // The position-table score_mod reads table[clip(i - j) + R] per pair: each stage
  // carries those entries for its 16 columns x 16 keys (clamped at copy time, four
  // more copies) beside K and V, so no vector read waits inside the loop; its ring has
  // one slot less to make room.
  constexpr bool kWin = SCORE == FA_S_RELPOS;
  constexpr int NS = kWin ? kStages - 1 : kStages;   // ring slots
  constexpr int WCP = kWin ? kDecCols * SK / 64 : 0;  // window copies per stage
  constexpr int CPSW = CPS + WCP;                     // copies per stage, window included
  using L = DLds<D, NS, kWin ? kDecCols * SK * 4 : 0>;
  static_assert(CPSW * (NS - 1) <= 63, "outstanding copies must fit the vmcnt counter");
  static_assert(NS >= 2 && NS <= 5, "the wait below spells out up to four stages in flight");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDecWaves * L::WAVE];

  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g4 = lane >> 4;

  const int ns = p.nsplit;
  // splits of one (b, h_kv) sit in one workgroup when ns divides kDecWaves: they are
  // merged through LDS at the end (no second kernel, no global partials)
  const bool local_merge = ns > 1 && kDecWaves % ns == 0;
  const int64_t units = (int64_t)p.B * p.Hkv * ns;
  const int64_t unit_raw = (int64_t)blockIdx.x * kDecWaves + w;
  const bool live = unit_raw < units;   // a trailing wave idles but still meets the barriers
  if (!live && !local_merge) return;    // wave-uniform; no barrier follows in this case
  const int64_t unit = live ? unit_raw : units - 1;
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

  // Q^T operand: lane holds Q[column][32 t + 8 g .. +8]
  bf16x8 qf[KT4];
  {
    const uint16_t* qrow = p.q + orow * D;
#pragma unroll
    for (int t = 0; t < KT4; ++t) {
      u32x4 v = col_ok ? load16(qrow + 32 * t + 8 * g4) : u32x4{0, 0, 0, 0};
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
  const int nst = live ? (e_end - e_begin) * (DKT / SK) : 0;
  // Each unit walks its stages starting at a unit-dependent rotation: units start at
  // the same offset of equally sized KV rows otherwise, and thousands of streams in
  // lockstep crowd the same HBM channels.  The online softmax is order-free.
  const int rot = nst > 0 ? (int)((unit * 37) % nst) : 0;
  auto rs = [&](int s) { const int t = s + rot; return t >= nst ? t - nst : t; };

  // first K/V row of this (b, h_kv) (contiguous layout), or the request's page-table
  // row (paged layout: logical key j lives in page pt_row[j >> page_shift], row
  // (page * Hkv + h_kv) * page_size + (j & (page_size - 1)) of the cache)
  const int hkv_m = hkv / p.kv_group;            // the KV head in memory
  const int Hkv_m = p.Hkv / p.kv_group;
  const int64_t krow0 = ((int64_t)b * Hkv_m + hkv_m) * p.kv_len;
  // The table is read through the constant address space at a wave-uniform index, so
  // the per-stage read is a scalar load, counted apart from the vector-memory copies
  // in flight (a vector read there makes the wait for it drain the copies as well).
  using cptr = const __attribute__((address_space(4))) int32_t*;
  const cptr pt_row = PAGED ? (cptr)sreg(p.pt + (int64_t)b * p.pt_stride) : nullptr;
  const int pshift = PAGED ? p.page_shift : 0;
  const int pmask = (1 << pshift) - 1;
  const int last_page = PAGED ? (int)(p.num_pages - 1) : 0;
  auto page_of = [&](int jb) -> int {
    // physical page of logical key jb (wave-uniform), clamped into the cache
    const int pg = pt_row[uniform(jb >> pshift)];
    return min(max(pg, 0), last_page);
  };
  auto row_of = [&](int jb, int pg) -> int64_t {
    if constexpr (PAGED) return ((int64_t)pg * Hkv_m + hkv_m) * (pmask + 1) + (jb & pmask);
    return krow0 + jb;
  };
  const int32_t* docr = doc_row(p.doc, b);
  int doc_i = (p.prog.has_doc && col_ok) ? docr[i_g] : 0;
  // consumed here: first used inside the stage loop, a load still counted as pending
  // there would make that use wait for all memory, copies in flight included
  asm volatile("" : "+v"(doc_i));
  // the keys' IDs are read as scalar loads (wave-uniform addresses in the constant
  // address space), counted apart from the copies
  const cptr docs = p.prog.has_doc ? (cptr)sreg(docr) : nullptr;
  const int doc_last = p.prog.has_doc ? (int)(p.doc.len - 1) : 0;
  const ScoreCtx sc = make_score_ctx(p.score, p.scale, hq);

  // the unit's block list, 64 entries per register (lane e holds entry base + e)
  int lst_base = 0;
  auto load_list = [&](int base) -> int {
    const int e = e_begin + base + lane;
    return e < e_end ? (e < nf ? flist[e] : plist[e - nf]) : 0;
  };
  int lst = load_list(0);
  // consume the loads here: the copies below are invisible to the compiler's wait
  // counting, which would otherwise wait for all memory at every use
#pragma unroll
  for (int t = 0; t < KT4; ++t) asm volatile("" : "+v"(qf[t]));
  asm volatile("" : "+v"(lst));
  auto stage_j0 = [&](int s) -> int {
    const int e = s / (DKT / SK);
    if (e - lst_base >= 64 || e < lst_base) {   // rare: other 64 entries (waits for all
      lst_base = e & ~63;                       // copies in flight)
      lst = load_list(lst_base);
    }
    return __builtin_amdgcn_readlane(lst, e - lst_base) * DKT + (s % (DKT / SK)) * SK;
  };
  auto stage_part = [&](int s) -> bool { return e_begin + s / (DKT / SK) >= nf; };

  // per-lane copy offsets (swizzles as in the prefill kernels)
  uint32_t koff[KVAR], voff[VVAR];
#pragma unroll
  for (int var = 0; var < KVAR; ++var) {
    const int key_in = lane / DCH;
    const int pc = lane % DCH;
    const int key = var * KPK + key_in;   // key within the swizzle period
    koff[var] = (uint32_t)(key_in * L::KROW + ((pc ^ k_swz<D>(key)) << 4));
    if (var < VVAR)
      voff[var] = (uint32_t)(key_in * L::KROW + ((2 * (((pc >> 1) ^ v_swz<D>(key)) & (L::UNITS - 1)) + (pc & 1)) << 4));
  }
  uint8_t* ring = smem + w * L::WAVE;
  const uint32_t ring_lds = lds_addr(ring);

  // table window: copy u fills entries 64 u + lane = 16 c + t (column c = 4 u + g4, key
  // j0 + t, t = col) from the centre of column c's table row (columns past the last
  // read column 0's)
  const int Rw = kWin ? p.score.radius : 0;
  const float* wtab[kWin ? WCP : 1];
  int wpos[kWin ? WCP : 1];
  if constexpr (kWin) {
#pragma unroll
    for (int u = 0; u < WCP; ++u) {
      const int c = 4 * u + g4 < ncols ? 4 * u + g4 : 0;
      const int hh_c = c / q_len;
      wtab[u] = p.score.table + (int64_t)(hkv * p.g + hh_c) * (2 * Rw + 1) + Rw;
      wpos[u] = c - hh_c * q_len + (int)p.q_offset;
    }
  }
  auto copy_window = [&](int j0, uint32_t mk) {
    if constexpr (kWin) {
      const uint32_t mw = mk + 2 * L::HALF;
#pragma unroll
      for (int u = 0; u < WCP; ++u) dma4_v(mw + 256 * u, wtab[u] + min(max(wpos[u] - (j0 + col), -Rw), Rw));
    }
  };

  // one stage (SK keys from j0) into ring slot `slot`; pg is the physical page of key
  // min(j0, kv_len - 1) (paged layout: a stage never crosses a page, and a ragged stage
  // only reads keys from that one up to kv_len - 1, inside the same page)
  auto copy_stage = [&](int j0, int pg, int slot) {
    const uint32_t mk = sreg(ring_lds + (uint32_t)slot * L::STAGE);
    const uint32_t mv = mk + L::HALF;
    if (j0 + SK <= kv_len) {
      const int64_t r0 = row_of(j0, pg);
      const char* kg = (const char*)p.k + r0 * L::KROW;
      const char* vg = (const char*)p.v + r0 * L::KROW;
      static_for<CPO>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int grp = (u / 4) * 4096;   // immediate offsets stay below 4 KB
        dma16_s_nt<(u % 4) * 1024>(mk + grp, kg + grp, koff[u % KVAR]);
        dma16_s_nt<(u % 4) * 1024>(mv + grp, vg + grp, voff[u % VVAR]);
      });
      copy_window(j0, mk);
    } else {
      // ragged tail: keys past kv_len re-read the last key (they are masked); offsets
      // from jb = min(j0, kv_len - 1) stay non-negative
      const int jb = min(j0, kv_len - 1);
      const int64_t rb = row_of(jb, pg);
      const char* kg = (const char*)p.k + rb * L::KROW;
      const char* vg = (const char*)p.v + rb * L::KROW;
      static_for<CPO>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const int key = u * KPK + lane / DCH;
        const uint32_t rowoff = (uint32_t)(min(j0 + key, kv_len - 1) - jb) * L::KROW;
        dma16_s_nt<0>(mk + u * 1024, kg, rowoff + (koff[u % KVAR] & (L::KROW - 1)));
        dma16_s_nt<0>(mv + u * 1024, vg, rowoff + (voff[u % VVAR] & (L::KROW - 1)));
      });
      copy_window(j0, mk);
    }
  };

  // per-lane LDS read bases.  K fragment t: key col, logical chunk 4t + g.  V^T
  // fragment dt: source row 4g + (col >> 2), head-dim 16 dt + 4 (col & 3).
  uint32_t kaddr[KT4], vaddr[DT];
#pragma unroll
  for (int t = 0; t < KT4; ++t) kaddr[t] = (uint32_t)k_off<D>(col, 4 * t + g4);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) vaddr[dt] = (uint32_t)v_off<D>(4 * g4 + (col >> 2), 16 * dt + 4 * (col & 3));

  float m_run = kNegInf;
  float l_run = 0.f;   // this lane's share; the four lane groups are summed at the end
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int j0, bool part, int slot) {
    const uint32_t so = (uint32_t)slot * L::STAGE;
    const uint8_t* kb = ring + so;
    const uint8_t* vb = kb + L::HALF;
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KT4; ++t) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kb + kaddr[t]);
      sacc = mfma16(__builtin_bit_cast(bf16x8, kv), qf[t], sacc);
    }
    // score_mod, then the mask (-inf) on partial and ragged stages only
    const int jl = j0 + 4 * g4;
    if constexpr (kWin) {
      const f32x4 tw = *reinterpret_cast<const f32x4*>(kb + 2 * L::HALF + (col * SK + 4 * g4) * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[r] = __builtin_fmaf(sacc[r], sc.c2, tw[r] * kLog2e);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[r] = score_log2<SCORE>(sacc[r], sc, i_g, jl + r);
    }
    if (part || j0 + SK > kv_len) {
      // the mask program over the lane's four keys at once, one bit per key
      auto span = [&](int lo, int hi) -> uint32_t {
        auto ge = [&](int a) -> uint32_t { return (0xFu << min(max(a, 0), 4)) & 0xFu; };
        return ge(lo - jl) & ~ge(hi - jl + 1);
      };
      uint32_t ok = span(0, kv_len - 1);
      if (part) {
        uint32_t db = 0;
        if (p.prog.has_doc) {
          const int js = uniform(j0);
          int d[SK];
#pragma unroll
          for (int x = 0; x < SK; ++x) d[x] = docs[min(js + x, doc_last)];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = g4 == 0 ? d[r] : (g4 == 1 ? d[4 + r] : (g4 == 2 ? d[8 + r] : d[12 + r]));
            db |= v == doc_i ? 1u << r : 0u;
          }
        }
        ok &= mask_word(p.prog, [&](int op, int a) { return row_leaf(op, a, i_g, span, db); });
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[r] = (ok >> r) & 1u ? sacc[r] : kNegInf;
    }
    float tmax = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    if (m_new > m_run) {
      const float alpha = fast_exp2(m_run - m_use);   // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    m_run = m_new;
    const float p0 = fast_exp2(sacc[0] - m_use);
    const float p1 = fast_exp2(sacc[1] - m_use);
    const float p2 = fast_exp2(sacc[2] - m_use);
    const float p3 = fast_exp2(sacc[3] - m_use);
    l_run += (p0 + p1) + (p2 + p3);
    const u32x2 pk = {cvt_pk_bf16(p0, p1), cvt_pk_bf16(p2, p3)};
    const s16x4 pb = __builtin_bit_cast(s16x4, pk);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vb + vaddr[dt]));
      oacc[dt] = mfma16k16(a, pb, oacc[dt]);
    }
  };

  // ring of NS slots: stage s in slot s % NS, the next NS - 1 in flight
  int issued = 0;
  int j0_of[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    j0_of[k] = 0;
    if (k < nst) {
      j0_of[k] = stage_j0(rs(k));
      copy_stage(j0_of[k], PAGED ? page_of(min(j0_of[k], kv_len - 1)) : 0, k);
      ++issued;
    }
  }
  int slot = 0;
  for (int s = 0; s < nst; ++s) {
    // stage s has landed once at most (issued - s - 1) stages of copies are outstanding
    switch (issued - s - 1) {
      case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(%0)" :: "i"(CPSW) : "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(%0)" :: "i"(2 * CPSW) : "memory"); break;
      case 3: asm volatile("s_waitcnt vmcnt(%0)" :: "i"(3 * CPSW) : "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(%0)" :: "i"(4 * CPSW) : "memory"); break;
    }
    int j0 = 0;
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (k == slot) j0 = j0_of[k];
    // the next stage's position (and its page, a scalar load that lands during the
    // compute below)
    const bool more = s + NS < nst;
    const int jn = more ? stage_j0(rs(s + NS)) : 0;
    const int pgn = (PAGED && more) ? page_of(min(jn, kv_len - 1)) : 0;
    compute(j0, stage_part(rs(s)), slot);
    if (more) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads of this slot are done
#pragma unroll
      for (int k = 0; k < NS; ++k)
        if (k == slot) j0_of[k] = jn;
      copy_stage(jn, pgn, slot);
      ++issued;
    }
    slot = slot + 1 == NS ? 0 : slot + 1;
  }

  // ---- results: final O and LSE (one split, or splits merged in LDS), or this
  // split's (m, l, o) partial for the merge kernel
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (local_merge) {
    // per wave: m[16], l[16], o[16][D] (columns x head dim), over the finished rings
    constexpr int RW = 32 + 16 * D;
    float* red = reinterpret_cast<float*>(smem);
    __syncthreads();
    float* mine = red + w * RW;
    if (g4 == 0) {
      mine[col] = m_run;
      mine[16 + col] = l_tot;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(mine + 32 + col * D + 16 * dt + 4 * g4) = oacc[dt];
    __syncthreads();
    if (!live || s_id != 0 || !col_ok) return;
    float M = kNegInf;
    for (int q = 0; q < ns; ++q) M = fmaxf(M, red[(w + q) * RW + col]);
    float wq[kDecWaves];
    float lsum = 0.f;
#pragma unroll
    for (int q = 0; q < kDecWaves; ++q) {
      wq[q] = 0.f;
      if (q < ns) {
        const float mq = red[(w + q) * RW + col];
        wq[q] = (mq == kNegInf) ? 0.f : fast_exp2(mq - M);
        lsum += wq[q] * red[(w + q) * RW + 16 + col];
      }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint16_t* o = p.o + orow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < kDecWaves; ++q)
        if (q < ns) acc += wq[q] * *reinterpret_cast<const f32x4*>(red + (w + q) * RW + 32 + col * D + 16 * dt + 4 * g4);
      u32x2 o2;
      o2[0] = cvt_pk_bf16(acc[0] * inv, acc[1] * inv);
      o2[1] = cvt_pk_bf16(acc[2] * inv, acc[3] * inv);
      *reinterpret_cast<u32x2*>(o + 16 * dt + 4 * g4) = o2;
    }
    if (g4 == 0) p.lse[orow] = lsum > 0.f ? (M + fast_log2(lsum)) * kLn2 : kNegInf;
    return;
  }
  if (!col_ok) return;
  if (ns == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* o = p.o + orow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x2 o2;
      o2[0] = cvt_pk_bf16(oacc[dt][0] * inv, oacc[dt][1] * inv);
      o2[1] = cvt_pk_bf16(oacc[dt][2] * inv, oacc[dt][3] * inv);
      *reinterpret_cast<u32x2*>(o + 16 * dt + 4 * g4) = o2;
    }
    if (g4 == 0) p.lse[orow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  } else {
    const int64_t rows = (int64_t)p.B * p.Hq * p.q_len;
    const int64_t prow = orow * ns + s_id;
    float* ws_m = p.ws;
    float* ws_l = p.ws + rows * ns;
    float* ws_o = p.ws + 2 * rows * ns;
    if (g4 == 0) {
      ws_m[prow] = m_run;
      ws_l[prow] = l_tot;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(ws_o + prow * D + 16 * dt + 4 * g4) = oacc[dt];
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

// The g query heads of a KV head share one walk over one table row, so their rows must
// be one row: tables broadcast over heads (H' = 1) or one query head per KV head.
bool decode_eligible(const FwdParams& p) {
  return p.tab.nqb == 1 && p.tab.bk == DKT && (int64_t)p.g * p.q_len <= kDecCols && p.q_len >= 1 &&
         (p.tab.tH == 1 || p.g == 1);
}

// Per-head tables under GQA (selector output picks blocks per query head): every query
// head becomes a unit of its own that walks its own row and reads its group's KV head,
// so the K/V of a group is read once per query head, as the different lists require.
bool decode_per_head(FwdParams& p) {
  if (p.tab.tH == 1 || p.g == 1 || p.kv_group != 1) return false;
  FwdParams v = p;
  v.kv_group = p.g;
  v.Hkv = p.Hq;
  v.g = 1;
  if (!decode_eligible(v)) return false;
  p = v;
  return true;
}

// splits per (b, h_kv): enough units for every wave slot (kDecWaves waves per CU, one
// workgroup per CU), capped by the listed block count of a row
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
  // one split, or splits merged inside a workgroup, write O and LSE directly
  if (nsplit <= 1 || kDecWaves % nsplit == 0) return 0;
  const size_t rows = (size_t)p.B * p.Hq * p.q_len;
  return rows * nsplit * (2 + (size_t)p.d) * sizeof(float);
}

namespace {

template <bool PAGED>
void launch_decode_kernel(const FwdParams& p, hipStream_t s, dim3 grid, dim3 block) {
#define FA_DEC(DD, SS) hipLaunchKernelGGL((decode_kernel<DD, SS, PAGED>), grid, block, 0, s, p)
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
}

}  // namespace

hipError_t launch_decode(const FwdParams& p, hipStream_t s) {
  const int64_t units = (int64_t)p.B * p.Hkv * p.nsplit;
  const dim3 grid((unsigned)((units + kDecWaves - 1) / kDecWaves));
  const dim3 block(64 * kDecWaves);
  if (p.pt) {
    launch_decode_kernel<true>(p, s, grid, block);
  } else {
    launch_decode_kernel<false>(p, s, grid, block);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit <= 1 || kDecWaves % p.nsplit == 0) return e;
  const int64_t rows = (int64_t)p.B * p.Hq * p.q_len;
  const dim3 cgrid((unsigned)((rows + 3) / 4));
  if (p.d == 128) hipLaunchKernelGGL((combine_kernel<128>), cgrid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((combine_kernel<64>), cgrid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
