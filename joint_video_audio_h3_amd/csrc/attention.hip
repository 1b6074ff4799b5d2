// Flash-style full attention over the packed sequence (gfx950, MFMA bf16).
//
//   o = softmax(q k^T / sqrt(d)) v   per head, over all n keys, no mask
// (minimax-h3-mlx README, "Architecture": full self-attention over the one
// packed sequence; "Performance": flash-style, the score matrix is never
// materialised).
//
// Two dense kernels share one design.  attn48_kernel (head_dim 128, the H3
// width) gives each wavefront 48 queries on 16x16x32 MFMAs, so every K or V^T
// fragment read from LDS feeds three MFMAs; it is described at its definition.
// attn_kernel (head_dim 96, and the block-sparse variant below) is described
// here.
//
// Work split: a block of 8 wavefronts takes 256 queries of one head; each
// wavefront owns 32 queries and walks all keys in tiles of 64, processed as
// two 32-key halves.  Blocks are dealt round-robin to the 8 XCDs; when the
// heads split evenly over them, block ids are remapped so that XCD x runs whole
// heads x, x+8, ..., and its L2 streams one head's K/V at a time.  A wave needs under 256 registers, so two waves share each
// SIMD and one's softmax runs beside the other's matrix work (VALU from one
// wave co-issues with the other's MFMAs).  K and V^T tiles stream HBM/L2 ->
// LDS with global_load_lds_dwordx4 into a 4-slot ring (three tiles in flight
// while one is consumed), XOR-swizzled so the 16-byte fragment reads are
// bank-conflict free.  The key loop is unrolled by the ring period so every
// slot offset is an immediate: loads take an SGPR tile base plus a fixed
// per-lane offset, fragment reads a per-lane base plus an immediate.
//
// Scores are computed transposed,  S^T[key][query] = K . Q^T  (MFMA A = K
// rows, B = Q fragment), so every lane holds one query (lane % 32) and 16 of
// its keys per 32-key half: K rows are read from LDS in a permuted order
// chosen so that accumulator register v of lane l holds key
// 16*(v/8) + 8*(l/32) + v%8, and the probabilities then already sit where the
// PV product wants its B operand:
//   O^T[dd][query] += V^T[dd][key] . P^T[key][query]
// with V^T written by the QKV epilogue (keys contiguous).  Both halves' score
// products are issued before the first half's softmax, so a wave's own matrix
// work runs under its exponentials.  Every 16-byte fragment read is issued a
// whole product (8 MFMAs) ahead of its use: a tile starts with the K fragments
// of its first half, and each MFMA of a product is paired with one read for the
// next (second half's K, then the V^T of each half).  One fragment per MFMA
// puts the LDS read port near its limit, so its latency has to be covered.
//
// Softmax: q arrives pre-scaled by log2(e)/sqrt(d), so scores are in log2
// units and p = exp2(s - m).  The reference point m of each query is folded
// into the score accumulator's initial value (-m).  No per-tile maximum is
// taken: p is rounded to bf16 for the PV product and summed from those bf16
// pairs (v_dot2), and only when some lane's 16 probabilities of a half sum
// above 2^8 (so that no p can exceed 2^8, or overflow) is the half's maximum
// formed, m raised, O and the running sum rescaled and p recomputed.  After
// the first tile this is rare.  The first half always sets m to its maximum
// (O and the sum are zero then, so nothing is rescaled).
// Keys at or beyond n are masked in the last tile; padded rows of q/k/v^T are
// zeros written by the QKV epilogue, so every operand is finite.
//
// Block-sparse variant (SPARSE): a block is one query tile of T = 64 or 128
// rows (T/32 wavefronts) and visits only the key tiles its CSR list selects
// for this head (FastH3 OmniRef (Ref2VA) on Apple Silicon MLX, "Opt-in M5
// attention backend": selected 64/128 tiles, only their valid rows).  A
// selected T-row tile is T/64 of the 64-key LDS tiles.  Blocks take a 2-slot
// ring (64 KB), so two blocks share a CU and their waves pair up per SIMD; the
// next selected tile loads while the current one is consumed.  Indices are
// clamped to the tile range, a list is cut at nq entries, and an empty list
// writes zeros.
#include <type_traits>

#include "h3_device.h"
#include "launch.h"

namespace h3 {

typedef __attribute__((address_space(3))) void* att_lds_t;
typedef __attribute__((address_space(3))) const bf16x8 att_lds_bf16x8_t;
typedef __bf16 att_bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t att_lds_addr(const void* p) { return (uint32_t)(uintptr_t)(att_lds_t)p; }
__device__ __forceinline__ bf16x8 att_read16(uint32_t a) { return *(att_lds_bf16x8_t*)(size_t)a; }
// 16 bytes per lane from sbase + voff (sbase wave-uniform) into LDS at lds + 16*lane
__device__ __forceinline__ void att_dma16s(uint32_t voff, const char* sbase, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void att_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int V>
using att_ic = std::integral_constant<int, V>;
// f(att_ic<0>), ..., f(att_ic<N-1>) in order, each index a compile-time constant
template <int I, int N, class F>
__device__ __forceinline__ void att_static_for_from(F&& f) {
  if constexpr (I < N) {
    f(att_ic<I>{});
    att_static_for_from<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void att_static_for(F&& f) {
  att_static_for_from<0, N>(f);
}

constexpr int ATT_WAVES = 8;            // wavefronts per block, 32 queries each (dense)
constexpr int ATT_BQ = ATT_WAVES * 32;  // queries per block (256, dense)
constexpr int ATT_BKV = 64;             // keys per tile
constexpr float ATT_RESCALE_SUM = 256.0f;   // a lane's 16 probabilities summing above 2^8

__device__ __forceinline__ int att_sigma(int i) {   // MFMA row -> key within 32
  const int g = i >> 3, h = (i >> 2) & 1, c = i & 3;
  return 16 * (g >> 1) + 8 * h + 4 * (g & 1) + c;
}
// K rows hold 16 chunks of 16 B; V^T rows 8 chunks.  Both swizzles depend only
// on the row modulo 32, so one per-lane base serves every 32-row tile.
__device__ __forceinline__ int att_kswz(int r) { return (r ^ (((r >> 3) & 1) << 2)) & 15; }
__device__ __forceinline__ int att_vswz(int r) { return ((r & 31) ^ ((r & 31) >> 3)) & 7; }

template <int HD, int W, bool SPARSE>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_kernel(AttnArgs p) {
  constexpr int ATT_SLOTS = SPARSE ? 2 : 4;   // LDS ring depth (tiles)
  constexpr int BQ = W * 32;                  // queries per block
  constexpr int DS = HD / 16;             // MFMA k-steps over head_dim
  constexpr int DT = HD / 32;             // 32-row tiles of head_dim in O^T
  constexpr int KROW = 256;               // LDS bytes per K row (16 chunks, HD/8 used)
  constexpr int VROW = ATT_BKV * 2;       // LDS bytes per V^T row (64 keys)
  constexpr int KBYTES = ATT_BKV * KROW;
  constexpr int VBYTES = HD * VROW;
  constexpr int STAGE = KBYTES + VBYTES;
  constexpr int NK = KBYTES / 1024, NV = VBYTES / 1024;   // 1 KB DMA loads per tile
  constexpr int NI = (NK + NV + W - 1) / W;               // per wavefront (last may idle)
  constexpr int NIK = NK / W;                             // first NIK loads are K
  static_assert(NK % W == 0, "K loads must split evenly over the waves");
  static_assert(ATT_SLOTS * STAGE <= 2 * 65536, "two 64 KB read windows");
  __shared__ __attribute__((aligned(1024))) char ring[ATT_SLOTS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // when the heads split evenly over the 8 XCDs (blocks are dealt to them
  // round-robin), XCD x takes whole heads x, x+8, ..., so its L2 streams one
  // head's K/V tiles at a time
  int qb = blockIdx.x, head = blockIdx.y;
  if (gridDim.y % 8 == 0) {
    const int id = blockIdx.x + gridDim.x * blockIdx.y;
    const int local = id / 8;
    qb = local % gridDim.x;
    head = id % 8 + 8 * (local / gridDim.x);
  }
  const int q0 = qb * BQ + wave * 32;
  const int hl = lane >> 5, lq = lane & 31;
  const size_t hoff = (size_t)head * p.n_pad * HD;

  // Q fragments (B operand): query q0 + lq, channels 16*ds + 8*hl .. +7
  bf16x8 qf[DS];
  {
    const uint16_t* qp = p.q + hoff + (size_t)(q0 + lq) * HD + 8 * hl;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ds] = *reinterpret_cast<const bf16x8*>(qp + ds * 16);
  }
  // Land the Q loads now (vmcnt(0) via the builtin, which the compiler's wait
  // bookkeeping understands): otherwise it keeps them "pending" into the key
  // loop and its vmcnt waits there would also wait for the K/V tiles in flight.
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));

  // DMA: K loads fill 4 rows of 256 B (lane -> row l/16, position l%16 holding
  // chunk (l%16)^kswz(row)); V^T loads fill 8 rows of 128 B (lane -> row l/8,
  // position l%8 holding chunk (l%8)^vswz(row)).  Offsets are relative to the
  // tile's first K row / first V^T column.
  const char* kbase0 = reinterpret_cast<const char*>(p.k + hoff);
  const char* vbase0 = reinterpret_cast<const char*>(p.vt + (size_t)head * HD * p.n_pad);
  const uint32_t ring0 = att_lds_addr(ring);
  uint32_t dvo[NI], dm[NI];
#pragma unroll
  for (int s = 0; s < NI; ++s) {
    const int j = min(wave + W * s, NK + NV - 1);
    if (s < NIK) {
      const int r = 4 * j + lane / 16;
      const int ch = min((lane & 15) ^ att_kswz(r), HD / 8 - 1);
      dvo[s] = (uint32_t)(r * HD + ch * 8) * 2;
      dm[s] = __builtin_amdgcn_readfirstlane(ring0 + j * 1024);
    } else {
      const int jv = j - NK;
      const int r = 8 * jv + lane / 8;
      const int ch = (lane & 7) ^ att_vswz(r);
      dvo[s] = (uint32_t)r * (uint32_t)p.n_pad * 2 + (uint32_t)ch * 16;
      dm[s] = __builtin_amdgcn_readfirstlane(ring0 + KBYTES + jv * 1024);
    }
  }
  const bool has_last = wave + W * (NI - 1) < NK + NV;   // wave-uniform: the last load exists
  // wait until at most T tiles of this wave's loads are in flight (a wave
  // without the last load issues NI - 1 per tile)
  auto wait_tiles = [&](auto T_) __attribute__((always_inline)) {
    constexpr int T = decltype(T_)::value;
    if constexpr ((NK + NV) % W == 0) {
      att_wait_vmcnt<T * NI>();
    } else {
      if (has_last) att_wait_vmcnt<T * NI>();
      else att_wait_vmcnt<T * (NI - 1)>();
    }
  };
  auto issue = [&](int kt, uint32_t slot_off) __attribute__((always_inline)) {
    const char* kb = kbase0 + (size_t)kt * (ATT_BKV * HD * 2);
    const char* vb = vbase0 + (size_t)kt * (ATT_BKV * 2);
#pragma unroll
    for (int s = 0; s < NI; ++s) {
      if (s == NI - 1 && !has_last) break;
      att_dma16s(dvo[s], s < NIK ? kb : vb, dm[s] + slot_off);
    }
  };

  // fragment read bases for two 64 KB windows of the ring
  const int krow = att_sigma(lq);
  const int kg = att_kswz(krow), vg = att_vswz(lq);
  uint32_t kbr[2][DS], vbr[2][4];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) kbr[w][ds] = ring0 + w * 65536 + krow * KROW + (((2 * ds + hl) ^ kg) * 16);
#pragma unroll
    for (int s = 0; s < 4; ++s) vbr[w][s] = ring0 + w * 65536 + lq * VROW + (((2 * s + hl) ^ vg) * 16);
  }
  // K fragment ds of half ks, V^T fragment (t, s) of the tile in the slot at
  // byte offset SO (compile-time, so the offset is an immediate)
  auto kread = [&](auto SO_, int ks, int ds) __attribute__((always_inline)) {
    constexpr int SO = decltype(SO_)::value;
    const int off = SO + ks * 32 * KROW;
    const int w = off >> 16;
    return att_read16(kbr[w][ds] + (off - (w << 16)));
  };
  auto vread = [&](auto SO_, int t, int s) __attribute__((always_inline)) {
    constexpr int SO = decltype(SO_)::value;
    const int off = SO + KBYTES + t * 32 * VROW;
    const int w = off >> 16;
    return att_read16(vbr[w][s] + (off - (w << 16)));
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_ref = 0.f, l_run = 0.f;
  const att_bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  const int KT = (p.n + ATT_BKV - 1) / ATT_BKV;

  // p = exp2(s) as bf16 pairs and their sum
  auto probs = [&](const f32x16& s, bf16x8 (&pf)[2]) __attribute__((always_inline)) {
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const att_bf16x2 pr = {(__bf16)__builtin_amdgcn_exp2f(s[v]), (__bf16)__builtin_amdgcn_exp2f(s[v + 1])};
      pf[v / 8][v % 8] = pr[0];
      pf[v / 8][v % 8 + 1] = pr[1];
      if ((v / 2) & 1) {
        rs1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs1, false);
      } else {
        rs0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs0, false);
      }
    }
    return rs0 + rs1;
  };
  // softmax of one half: probabilities into pf, running sum updated; the rare
  // rescale also shifts `other`, the other half's scores already formed with
  // the old reference point
  auto softmax = [&](f32x16& s, auto&& shift_other, bool first, bf16x8 (&pf)[2]) __attribute__((always_inline)) {
    float rs = probs(s, pf);
    if (first || __builtin_amdgcn_ballot_w64(!(rs <= ATT_RESCALE_SUM)) != 0) {
      float mx = s[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float sh = first ? mx : fmaxf(mx, 0.f);
      m_ref += sh;
      // O and the running sum are still zero on the first half: nothing to
      // rescale (and exp2(-sh) would overflow when every first score is far
      // below zero)
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(-sh);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] -= sh;
      shift_other(sh);
      rs = probs(s, pf);
    }
    l_run += rs;
  };
  auto mask = [&](f32x16& s, int key0) __attribute__((always_inline)) {
    if (key0 + 32 > p.n) {   // only the last tile can hold keys >= n
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (key0 + 16 * (v / 8) + 8 * hl + (v % 8) >= p.n) s[v] = -INFINITY;
    }
  };

  // one tile: S^T = K Q^T - m for both halves, then each half's softmax and
  // O^T += V^T P^T.  Fragment reads run a whole product ahead: the K fragments
  // of half 0 first, then each MFMA of a product is paired with one read for the
  // next product (half 1's K, then half 0's V^T, then half 1's V^T)
  auto tile_body = [&](auto&& kr, auto&& vr, int kt, bool masked, bool first) __attribute__((always_inline)) {
    bf16x8 ka[DS], kb[DS], va[2 * DT], vb[2 * DT];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) ka[ds] = kr(0, ds);
    f32x16 s0, s1;
#pragma unroll
    for (int v = 0; v < 16; ++v) s0[v] = -m_ref;
    s1 = s0;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      s0 = mfma32(ka[ds], qf[ds], s0);
      kb[ds] = kr(1, ds);
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      s1 = mfma32(kb[ds], qf[ds], s1);
      va[ds] = vr(ds / 2, ds % 2);
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (masked) {
      mask(s0, kt * ATT_BKV);
      mask(s1, kt * ATT_BKV + 32);
    }
    bf16x8 pf[2];
    // each softmax at low wave priority, the MFMA runs at high (as attn48_kernel)
    __builtin_amdgcn_s_setprio(0);
    softmax(s0, [&](float sh) __attribute__((always_inline)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s1[v] -= sh;
    }, first, pf);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 2 * DT; ++i) {
      oacc[i / 2] = mfma32(va[i], pf[i % 2], oacc[i / 2]);
      vb[i] = vr(i / 2, 2 + i % 2);
    }
    __builtin_amdgcn_s_setprio(0);
    softmax(s1, [](float) {}, false, pf);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 2 * DT; ++i) oacc[i / 2] = mfma32(vb[i], pf[i % 2], oacc[i / 2]);
  };

  // steady tile with compile-time slot U: wait for tile kt, barrier, refill the
  // slot freed by tile kt-1 with tile kt+3, consume tile kt
  auto tile_c = [&](auto U_, int kt) __attribute__((always_inline)) {
    constexpr int U = decltype(U_)::value;
    constexpr int SO = U * STAGE;
    wait_tiles(att_ic<2>{});
    __builtin_amdgcn_s_barrier();
    issue(kt + 3, (uint32_t)(((U + 3) % ATT_SLOTS) * STAGE));
    tile_body([&](int ks, int ds) __attribute__((always_inline)) { return kread(att_ic<SO>{}, ks, ds); },
              [&](int t, int s) __attribute__((always_inline)) { return vread(att_ic<SO>{}, t, s); }, kt, false,
              kt == 0);
  };
  // the same with the slot from the runtime phase (the last few tiles)
  auto tile_r = [&](int kt) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)((kt % ATT_SLOTS) * STAGE);
    if (kt + 2 < KT) {
      wait_tiles(att_ic<2>{});
    } else if (kt + 1 < KT) {
      wait_tiles(att_ic<1>{});
    } else {
      att_wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (kt + 3 < KT) issue(kt + 3, (uint32_t)(((kt + 3) % ATT_SLOTS) * STAGE));
    tile_body([&](int ks, int ds) __attribute__((always_inline)) { return att_read16(kbr[0][ds] + so + ks * 32 * KROW); },
              [&](int t, int s) __attribute__((always_inline)) { return att_read16(vbr[0][s] + so + KBYTES + t * 32 * VROW); },
              kt, kt + 1 == KT, kt == 0);
  };

  if constexpr (!SPARSE) {
    issue(0, 0);
    if (KT > 1) issue(1, STAGE);
    if (KT > 2) issue(2, 2 * STAGE);
    int kt = 0;
    for (; kt + 7 <= KT; kt += 4) {   // the last of the four issues tile kt + 6
      tile_c(att_ic<0>{}, kt);
      tile_c(att_ic<1>{}, kt + 1);
      tile_c(att_ic<2>{}, kt + 2);
      tile_c(att_ic<3>{}, kt + 3);
    }
    for (; kt < KT; ++kt) tile_r(kt);
  } else {
    // the selected key tiles of this (head, query tile), as 64-key LDS tiles
    constexpr int R = BQ / ATT_BKV;             // 64-key tiles per selected tile (1 or 2)
    const int nq = (p.n + BQ - 1) / BQ;
    const int* sel = p.tile_idx + p.tile_off[head * nq + qb];
    // a list holds at most nq distinct tiles: a longer (malformed) one is cut there
    const int cnt = min(max(p.tile_off[head * nq + qb + 1] - p.tile_off[head * nq + qb], 0), nq);
    const int nkv = cnt * R;
    auto kv_of = [&](int i) __attribute__((always_inline)) {
      const int j = min(max(sel[i / R], 0), nq - 1);
      return j * R + i % R;
    };
    // tile i in slot U (compile-time): wait for it, barrier (every wave's part
    // landed, tile i-1 consumed), start tile i+1 in the other slot, consume i
    auto tile_s = [&](auto U_, int i, int kv) __attribute__((always_inline)) {
      constexpr int U = decltype(U_)::value;
      constexpr int SO = U * STAGE;
      att_wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (i + 1 < nkv) issue(kv_of(i + 1), (uint32_t)((1 - U) * STAGE));
      tile_body([&](int ks, int ds) __attribute__((always_inline)) { return kread(att_ic<SO>{}, ks, ds); },
                [&](int t, int s) __attribute__((always_inline)) { return vread(att_ic<SO>{}, t, s); }, kv,
                kv + 1 >= KT, i == 0);
    };
    if (nkv > 0) issue(kv_of(0), 0);
    for (int i = 0; i < nkv; i += 2) {
      tile_s(att_ic<0>{}, i, kv_of(i));
      if (i + 1 < nkv) tile_s(att_ic<1>{}, i + 1, kv_of(i + 1));
    }
  }

  const float lsum = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;   // an empty selection writes zeros
  const int qrow = q0 + lq;
  if (qrow < p.n) {
    uint16_t* op = p.o + (size_t)qrow * p.heads * HD + head * HD;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = t * 32 + 8 * g + 4 * hl;
        const f32x16& a = oacc[t];
        const uint2 w = make_uint2(pack2bf(a[4 * g] * inv, a[4 * g + 1] * inv),
                                   pack2bf(a[4 * g + 2] * inv, a[4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(op + dd) = w;
      }
  }
}

// ============================================================ dense, head_dim 128: 48 queries per wave
// The same ring, DMA, XCD mapping and lazy-rescale softmax as attn_kernel, on
// v_mfma_f32_16x16x32_bf16 with 48 queries (three groups of 16) per wavefront:
// every K or V^T fragment read from LDS feeds three MFMAs, one per query group,
// so a key costs two thirds of the LDS reads it costs with one 32-query group
// per fragment, at about the same register count (two waves per SIMD).
//   A (16 x 32): lane l holds row l%16, k elements 8*(l/16) .. +7
//   B (32 x 16): lane l holds column l%16, k elements 8*(l/16) .. +7
//   D (16 x 16): lane l holds rows 4*(l/16) .. +3 of column l%16
// Scores are S^T = K Q^T in 16-key slices: A = K rows, B = Q^T of a group.  A
// 32-key half is two slices, and slice j's A row r reads key
// 8*(r/4) + 4*j + r%4, so the lane holding D rows 4g .. 4g+3 of both slices
// holds keys 8g .. 8g+7 of its query: exactly the k elements of P^T that the
// product O^T += V^T P^T takes as its B operand, with V^T's A fragment reading
// keys 8*(l/16) .. +7.  Each query's softmax state lives in the four lanes
// l%16 of its group and is kept equal in them.
constexpr int A48_QW = 48;                   // queries per wavefront
constexpr int A48_WAVES = 8;
constexpr int A48_BQ = A48_WAVES * A48_QW;   // queries per block

__device__ __forceinline__ f32x4 a48_mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// key (within a 32-key half) read by A row r of score slice j
__device__ __forceinline__ int a48_krow(int j, int r) { return 8 * (r >> 2) + 4 * j + (r & 3); }
// A 16-byte LDS read takes 16 lanes (256 bytes, all 64 banks) per cycle, so
// each 16-lane group of a fragment read must touch 16 distinct 16-byte bank
// groups (and, then, each 8-lane half 8 distinct ones modulo 8).
// K rows (256 bytes = 16 chunks): chunk c at position c ^ a48_kswz(row).  The
// 16 rows of a fragment's 16 lanes differ in bits 0, 1, 3 and 4, which this
// maps to 16 distinct positions.
__device__ __forceinline__ int a48_kswz(int r) { return (r & 3) | ((r >> 1) & 12); }
// V^T rows (64 keys = 8 chunks, two rows per 256 bytes): chunk c at position
// c ^ a48_vswz(row); 16 consecutive rows land on 16 distinct bank groups, and 8
// consecutive rows on 8 distinct positions.
__device__ __forceinline__ int a48_vswz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

__global__ __launch_bounds__(A48_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn48_kernel(
    AttnArgs p) {
  constexpr int HD = 128, W = A48_WAVES, SLOTS = 4;
  constexpr int DC = HD / 32;              // 32-wide d chunks (score product k steps)
  constexpr int DT = HD / 16;              // 16-row d tiles of O^T
  constexpr int NG = A48_QW / 16;          // query groups per wave
  constexpr int KROW = 256, VROW = ATT_BKV * 2;
  constexpr int KBYTES = ATT_BKV * KROW, VBYTES = HD * VROW, STAGE = KBYTES + VBYTES;
  constexpr int NK = KBYTES / 1024, NV = VBYTES / 1024;
  constexpr int NIK = NK / W, NI = (NK + NV) / W;
  static_assert(NK % W == 0 && NV % W == 0, "loads split evenly over the waves");
  // the K tiles of all slots fill the first 64 KB of the ring and the V^T tiles
  // the second, so every fragment read is a per-lane base plus an immediate
  // below 64 KB; a slot's K and V^T tiles sit at the same offset in their halves
  static_assert(KBYTES == 16384 && VBYTES == 16384 && SLOTS * KBYTES == 65536, "ring halves");
  __shared__ __attribute__((aligned(1024))) char ring[SLOTS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int qb = blockIdx.x, head = blockIdx.y;
  if (gridDim.y % 8 == 0) {   // XCD x runs whole heads x, x+8, ... (as attn_kernel)
    const int id = blockIdx.x + gridDim.x * blockIdx.y;
    const int local = id / 8;
    qb = local % gridDim.x;
    head = id % 8 + 8 * (local / gridDim.x);
  }
  const int q0 = qb * A48_BQ + wave * A48_QW;
  const int lr = lane & 15, lg = lane >> 4;
  const size_t hoff = (size_t)head * p.n_pad * HD;

  // Q^T fragments (B operand): query q0 + 16*gr + lr, channels 32*dc + 8*lg .. +7
  // (rows past n_pad, in the last block, read row n_pad - 1; their outputs are not stored)
  bf16x8 qf[DC][NG];
#pragma unroll
  for (int gr = 0; gr < NG; ++gr) {
    const uint16_t* qp = p.q + hoff + (size_t)min(q0 + 16 * gr + lr, p.n_pad - 1) * HD + 8 * lg;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc][gr] = *reinterpret_cast<const bf16x8*>(qp + 32 * dc);
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0): see attn_kernel

  // DMA: K load j fills rows 4j .. 4j+3 (lane -> row l/16, position l%16 holding
  // chunk (l%16) ^ kswz(row)); V^T load j fills d rows 8j .. 8j+7 (lane -> row
  // l/8, position l%8 holding key chunk (l%8) ^ vswz(row))
  const char* kbase0 = reinterpret_cast<const char*>(p.k + hoff);
  const char* vbase0 = reinterpret_cast<const char*>(p.vt + (size_t)head * HD * p.n_pad);
  const uint32_t ring0 = att_lds_addr(ring);
  uint32_t dvo[NI], dm[NI];
#pragma unroll
  for (int s = 0; s < NI; ++s) {
    const int j = wave + W * s;
    if (s < NIK) {
      const int r = 4 * j + lane / 16;
      dvo[s] = (uint32_t)(r * HD + ((lane & 15) ^ a48_kswz(r)) * 8) * 2;
      dm[s] = __builtin_amdgcn_readfirstlane(ring0 + j * 1024);
    } else {
      const int jv = j - NK;
      const int r = 8 * jv + lane / 8;
      dvo[s] = (uint32_t)r * (uint32_t)p.n_pad * 2 + (uint32_t)(((lane & 7) ^ a48_vswz(r)) * 16);
      dm[s] = __builtin_amdgcn_readfirstlane(ring0 + 65536 + jv * 1024);
    }
  }
  auto issue = [&](int kt, uint32_t slot_off) __attribute__((always_inline)) {
    const char* kb = kbase0 + (size_t)kt * (ATT_BKV * HD * 2);
    const char* vb = vbase0 + (size_t)kt * (ATT_BKV * 2);
#pragma unroll
    for (int s = 0; s < NI; ++s) att_dma16s(dvo[s], s < NIK ? kb : vb, dm[s] + slot_off);
  };

  // fragment read bases: K for d chunk dc, V^T for half h; the slot, the half's
  // key offset, the slice (its rows are slice 0's plus 4, with the same
  // swizzle: a48_krow(0, r) has bit 2 clear) and the d tile are immediates
  uint32_t kbr[DC], vbr[2];
  {
    const int r = a48_krow(0, lr);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kbr[dc] = ring0 + r * KROW + (((4 * dc + lg) ^ a48_kswz(r)) * 16);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) vbr[h] = ring0 + 65536 + lr * VROW + (((4 * h + lg) ^ a48_vswz(lr)) * 16);
  // fragment u of a tile in the slot at offset SO (of each half of the ring):
  // u = 16h + f, f < 8 the K fragment of slice f/4, chunk f%4 of half h; f >= 8
  // the V^T fragment of d tile f-8 of half h
  auto fread = [&](auto SO_, auto U_) __attribute__((always_inline)) {
    constexpr int SO = decltype(SO_)::value, U = decltype(U_)::value;
    constexpr int H = U / 16, F = U % 16;
    if constexpr (F < 8) return att_read16(kbr[F % 4] + (SO + H * 32 * KROW + (F / 4) * 4 * KROW));
    else return att_read16(vbr[H] + (SO + (F - 8) * 16 * VROW));
  };
  auto fread_rt = [&](uint32_t so, auto U_) __attribute__((always_inline)) {
    constexpr int U = decltype(U_)::value;
    constexpr int H = U / 16, F = U % 16;
    if constexpr (F < 8) return att_read16(kbr[F % 4] + so + (H * 32 * KROW + (F / 4) * 4 * KROW));
    else return att_read16(vbr[H] + so + (F - 8) * 16 * VROW);
  };

  f32x4 oacc[DT][NG];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) oacc[t][gr] = f32x4{};
  // -m of each query (its reference point, replicated in a 4-register tuple):
  // the C operand of the first MFMA of every score slice, so scores come out
  // relative to m with no per-half initialisation
  f32x4 mneg[NG];
  float l_run[NG];
#pragma unroll
  for (int gr = 0; gr < NG; ++gr) {
    mneg[gr] = f32x4{};
    l_run[gr] = 0.f;
  }
  const att_bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int KT = (p.n + ATT_BKV - 1) / ATT_BKV;

  // p = exp2(s) for a group's 8 scores (slice j, row i -> k element 4j + i) as
  // bf16 and the sum of those bf16 values
  auto probs = [&](const f32x4 (&s)[2], bf16x8& pf) __attribute__((always_inline)) {
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const att_bf16x2 pr = {(__bf16)__builtin_amdgcn_exp2f(s[j][i]), (__bf16)__builtin_amdgcn_exp2f(s[j][i + 1])};
        pf[4 * j + i] = pr[0];
        pf[4 * j + i + 1] = pr[1];
        rs = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs, false);
      }
    return rs;
  };
  // the half's softmax (scores sc[gr][j], already relative to m): the
  // probabilities into pf, the running sums updated; rarely (some lane's 8
  // probabilities of a group sum above 2^8, or the first half) the half's
  // maximum of each query is formed, m raised, O and the sum rescaled
  auto softmax = [&](f32x4 (&sc)[NG][2], bf16x8 (&pf)[NG], bool first) __attribute__((always_inline)) {
    float rs[NG];
    bool big = false;
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) {
      rs[gr] = probs(sc[gr], pf[gr]);
      big |= !(rs[gr] <= ATT_RESCALE_SUM);
    }
    if (first || __builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) {
        float mx = sc[gr][0][0];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[gr][j][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float sh = first ? mx : fmaxf(mx, 0.f);
        mneg[gr] -= sh;
        if (!first) {   // (first: O and the sum are still zero)
          const float alpha = __builtin_amdgcn_exp2f(-sh);
          l_run[gr] *= alpha;
#pragma unroll
          for (int t = 0; t < DT; ++t) oacc[t][gr] *= alpha;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[gr][j][i] -= sh;
        rs[gr] = probs(sc[gr], pf[gr]);
      }
    }
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) l_run[gr] += rs[gr];
  };

  // One tile: per 32-key half, the score product (8 K fragments x 3 query
  // groups), its softmax, then O^T += V^T P^T (8 V^T fragments x 3 groups).
  // Fragment reads run PD fragments ahead of their MFMAs.
  constexpr int PD = 3;
  auto tile_body = [&](auto&& rd, int kt, bool masked, bool first) __attribute__((always_inline)) {
    bf16x8 fr[PD + 1];
    f32x4 sc[NG][2];
    bf16x8 pf[NG];
    att_static_for<PD>([&](auto U_) __attribute__((always_inline)) {
      constexpr int U = decltype(U_)::value;
      fr[U] = rd(att_ic<U>{});
    });
    att_static_for<32>([&](auto U_) __attribute__((always_inline)) {
      constexpr int U = decltype(U_)::value;
      constexpr int H = U / 16, F = U % 16;
      if constexpr (F == 8) {
        if (masked) {   // only the last tile holds keys >= n
          const int key0 = kt * ATT_BKV + 32 * H + 8 * lg;
#pragma unroll
          for (int gr = 0; gr < NG; ++gr)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (key0 + 4 * j + i >= p.n) sc[gr][j][i] = -INFINITY;
        }
        // the softmax at low wave priority, the MFMA runs at high: while one wave
        // of a SIMD works through its softmax, the other's MFMAs win the issue
        // port (measured 1.8 % faster at 49,840 rows)
        __builtin_amdgcn_s_setprio(0);
        softmax(sc, pf, first && H == 0);
        __builtin_amdgcn_s_setprio(1);
      }
      if constexpr (U + PD < 32) fr[(U + PD) % (PD + 1)] = rd(att_ic<U + PD>{});
      const bf16x8& a = fr[U % (PD + 1)];
      if constexpr (F < 8) {
#pragma unroll
        for (int gr = 0; gr < NG; ++gr)
          sc[gr][F / 4] = a48_mfma(a, qf[F % 4][gr], F % 4 == 0 ? mneg[gr] : sc[gr][F / 4]);
      } else {
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) oacc[F - 8][gr] = a48_mfma(a, pf[gr], oacc[F - 8][gr]);
      }
    });
  };

  auto wait_tiles = [&](auto T_) __attribute__((always_inline)) { att_wait_vmcnt<decltype(T_)::value * NI>(); };
  // steady tile with compile-time slot U (as attn_kernel)
  auto tile_c = [&](auto U_, int kt) __attribute__((always_inline)) {
    constexpr int U = decltype(U_)::value;
    constexpr int SO = U * KBYTES;
    wait_tiles(att_ic<2>{});
    __builtin_amdgcn_s_barrier();
    issue(kt + 3, (uint32_t)(((U + 3) % SLOTS) * KBYTES));
    tile_body([&](auto F_) __attribute__((always_inline)) { return fread(att_ic<SO>{}, F_); }, kt, false, kt == 0);
  };
  auto tile_r = [&](int kt) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)((kt % SLOTS) * KBYTES);
    if (kt + 2 < KT) {
      wait_tiles(att_ic<2>{});
    } else if (kt + 1 < KT) {
      wait_tiles(att_ic<1>{});
    } else {
      att_wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (kt + 3 < KT) issue(kt + 3, (uint32_t)(((kt + 3) % SLOTS) * KBYTES));
    tile_body([&](auto F_) __attribute__((always_inline)) { return fread_rt(so, F_); }, kt, kt + 1 == KT, kt == 0);
  };

  issue(0, 0);
  if (KT > 1) issue(1, KBYTES);
  if (KT > 2) issue(2, 2 * KBYTES);
  int kt = 0;
  for (; kt + 7 <= KT; kt += 4) {
    tile_c(att_ic<0>{}, kt);
    tile_c(att_ic<1>{}, kt + 1);
    tile_c(att_ic<2>{}, kt + 2);
    tile_c(att_ic<3>{}, kt + 3);
  }
  for (; kt < KT; ++kt) tile_r(kt);

#pragma unroll
  for (int gr = 0; gr < NG; ++gr) {
    float lsum = l_run[gr] + __shfl_xor(l_run[gr], 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    const int qrow = q0 + 16 * gr + lr;
    if (qrow < p.n) {
      uint16_t* op = p.o + (size_t)qrow * p.heads * HD + head * HD + 4 * lg;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const f32x4& a = oacc[t][gr];
        *reinterpret_cast<uint2*>(op + 16 * t) =
            make_uint2(pack2bf(a[0] * inv, a[1] * inv), pack2bf(a[2] * inv, a[3] * inv));
      }
    }
  }
}

template <int HD>
static hipError_t launch_hd(const AttnArgs& a, hipStream_t s) {
  if (!a.tile_idx) {
    if constexpr (HD == 128) {
      attn48_kernel<<<dim3((a.n + A48_BQ - 1) / A48_BQ, a.heads), A48_WAVES * 64, 0, s>>>(a);
    } else {
      attn_kernel<HD, ATT_WAVES, false><<<dim3((a.n + ATT_BQ - 1) / ATT_BQ, a.heads), ATT_WAVES * 64, 0, s>>>(a);
    }
  } else if (a.tile == 128) {
    attn_kernel<HD, 4, true><<<dim3((a.n + 127) / 128, a.heads), 256, 0, s>>>(a);
  } else if (a.tile == 64) {
    // two waves per block and two 64 KB blocks per CU: one wave per SIMD whatever
    // the register count (the build notes that two per SIMD is not reached)
    attn_kernel<HD, 2, true><<<dim3((a.n + 63) / 64, a.heads), 128, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.head_dim == 128) return launch_hd<128>(a, s);
  if (a.head_dim == 96) return launch_hd<96>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace h3
