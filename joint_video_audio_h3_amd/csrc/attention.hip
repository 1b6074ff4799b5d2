// Flash-style full attention over the packed sequence (gfx950, MFMA bf16).
//
//   o = softmax(q k^T / sqrt(d)) v   per head, over all n keys, no mask
// (minimax-h3-mlx README, "Architecture": full self-attention over the one
// packed sequence; "Performance": flash-style, the score matrix is never
// materialised).
//
// Work split: a block of ATT_WAVES wavefronts takes 256 queries of one head;
// each wavefront owns ATT_QS sub-tiles of 32 queries (sub-tiles of one wave
// share every K and V fragment it reads from LDS) and walks all keys in tiles
// of 64, processed as two 32-key halves.  With 8 waves x 32 queries a wave
// needs ~170 registers, so two waves share each SIMD and one's softmax hides
// behind the other's matrix work.  K and V^T tiles stream HBM/L2 -> LDS with
// global_load_lds_dwordx4 into a 3-slot ring (two tiles in flight while one is
// consumed), XOR-swizzled so the 16-byte fragment reads are bank-conflict free.
//
// Scores are computed transposed,  S^T[key][query] = K . Q^T  (MFMA A = K
// rows, B = Q fragment), so every lane holds one query (lane % 32) and 16 of
// its keys per 32-key sub-tile: the running max and sum need only the two
// half-waves combined.  K rows are read from LDS in a permuted order chosen so
// that accumulator register v of lane l holds key 16*(v/8) + 8*(l/32) + v%8;
// the probabilities then already sit where the PV product wants its B operand:
//   O^T[dd][query] += V^T[dd][key] . P^T[key][query]
// with V^T written by the QKV epilogue (keys contiguous).
//
// Softmax: q arrives pre-scaled by log2(e)/sqrt(d), so scores are in log2
// units and p = exp2(s - m).  The reference point m of each query is folded
// into the score accumulator's initial value (-m), and it is only raised when
// a tile's scores exceed it by more than 8 (p <= 2^8, exact in fp32 and bf16
// relative precision), so rescaling O is rare.  Row sums are fp32 per lane.
// Keys at or beyond n are masked in the last tile; padded rows of q/k/v^T are
// zeros written by the QKV epilogue, so every operand is finite.
#include "h3_device.h"
#include "launch.h"

namespace h3 {

typedef __attribute__((address_space(3))) void* att_lds_t;

__device__ __forceinline__ void att_dma16(const void* g, void* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(att_lds_t)lds;
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(la) : "memory");
}
template <int N>
__device__ __forceinline__ void att_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

constexpr int ATT_WAVES = 8;   // wavefronts per block
constexpr int ATT_QS = 1;      // 32-query sub-tiles per wavefront
constexpr int ATT_BQ = ATT_WAVES * 32 * ATT_QS;   // queries per block (256)
constexpr int ATT_BKV = 64;    // keys per tile
constexpr float ATT_RESCALE = 8.0f;   // raise m only when scores exceed it by > 2^8

__device__ __forceinline__ int att_sigma(int i) {   // MFMA row -> key within 32
  const int g = i >> 3, h = (i >> 2) & 1, c = i & 3;
  return 16 * (g >> 1) + 8 * h + 4 * (g & 1) + c;
}
__device__ __forceinline__ int att_kswz(int r) { return (r ^ (((r >> 3) & 1) << 2)) & 15; }
__device__ __forceinline__ int att_vswz(int r) { return (r ^ (r >> 3)) & 7; }

template <int HD>
__global__ __launch_bounds__(ATT_WAVES * 64) void attn_kernel(AttnArgs p) {
  constexpr int DS = HD / 16;             // MFMA k-steps over head_dim
  constexpr int DT = HD / 32;             // 32-row tiles of head_dim in O^T
  constexpr int KROW = 256;               // LDS bytes per K row (16 chunks, HD/8 used)
  constexpr int VROW = ATT_BKV * 2;       // LDS bytes per V^T row (64 keys)
  constexpr int KBYTES = ATT_BKV * KROW;
  constexpr int VBYTES = HD * VROW;
  constexpr int STAGE = KBYTES + VBYTES;
  constexpr int NK = KBYTES / 1024, NV = VBYTES / 1024;   // 1 KB DMA loads per tile
  constexpr int W = ATT_WAVES, QS = ATT_QS;
  constexpr int NI = (NK + NV + W - 1) / W;               // per wavefront (last may idle)
  constexpr int NIK = NK / W;                             // first NIK slots load K
  static_assert(NK % W == 0, "K loads must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char ring[3 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  const int q0 = blockIdx.x * ATT_BQ + wave * 32 * QS;
  const int hl = lane >> 5, lq = lane & 31;
  const size_t hoff = (size_t)head * p.n_pad * HD;

  // Q fragments (B operand): query q0 + 32*qs + lq, channels 16*ds + 8*hl .. +7
  bf16x8 qf[QS][DS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const uint16_t* qp = p.q + hoff + (size_t)(q0 + qs * 32 + lq) * HD + 8 * hl;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[qs][ds] = *reinterpret_cast<const bf16x8*>(qp + ds * 16);
  }
  // Land the Q loads now (vmcnt(0) via the builtin, which the compiler's wait
  // bookkeeping understands): otherwise it keeps them "pending" into the key
  // loop and its vmcnt waits there would also wait for the K/V tiles in flight.
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));

  // DMA sources: K slots fill 4 rows of 256 B per load (lane -> row l/16,
  // position l%16 holding chunk (l%16)^kswz(row)); V^T slots fill 8 rows of
  // 128 B (lane -> row l/8, position l%8 holding chunk (l%8)^vswz(row)).
  const uint16_t* src[NI];
  int ldso[NI];
#pragma unroll
  for (int s = 0; s < NI; ++s) {
    const int j = min(wave + W * s, NK + NV - 1);   // idle slots repeat a valid load
    if (s < NIK) {
      const int r = 4 * j + lane / 16;
      const int ch = min((lane & 15) ^ att_kswz(r), HD / 8 - 1);
      src[s] = p.k + hoff + (size_t)r * HD + ch * 8;
      ldso[s] = j * 1024;
    } else {
      const int jv = j - NK;
      const int r = 8 * jv + lane / 8;
      const int ch = (lane & 7) ^ att_vswz(r);
      src[s] = p.vt + (size_t)head * HD * p.n_pad + (size_t)r * p.n_pad + ch * 8;
      ldso[s] = KBYTES + jv * 1024;
    }
  }
  auto issue = [&](int kt, char* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < NI; ++s) {
      if (wave + W * s >= NK + NV) break;   // wave-uniform: this slot has no load
      const size_t step = s < NIK ? (size_t)ATT_BKV * HD : (size_t)ATT_BKV;
      att_dma16(src[s] + kt * step, buf + ldso[s]);
    }
  };

  // fragment read offsets
  const int krow = att_sigma(lq);
  const int koff = krow * KROW;
  const int kg = att_kswz(krow);
  int voff[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) voff[t] = KBYTES + (t * 32 + lq) * VROW;
  int vg[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) vg[t] = att_vswz(t * 32 + lq);

  f32x16 oacc[DT][QS];
  float m_ref[QS], l_run[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t][qs] = f32x16{};
    m_ref[qs] = l_run[qs] = 0.f;
  }

  const int KT = (p.n + ATT_BKV - 1) / ATT_BKV;

  // one 32-key half of a tile: scores, softmax bookkeeping, PV accumulation
  auto half_tile = [&](int kt, int ks, const char* buf) __attribute__((always_inline)) {
    const bool first = kt == 0 && ks == 0;
    // ---- S^T = K Q^T - m   (both query sub-tiles share each K fragment)
    f32x16 sacc[QS];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const float init = first ? 0.f : -m_ref[qs];
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[qs][v] = init;
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          buf + ks * 32 * KROW + koff + (((2 * ds + hl) ^ kg) * 16));
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) sacc[qs] = mfma32(a, qf[qs][ds], sacc[qs]);
    }
    const int key0 = kt * ATT_BKV + ks * 32;
    if (key0 + 32 > p.n) {   // only the last keys can be padding: mask keys >= n
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + 16 * (v / 8) + 8 * hl + (v % 8);
        if (key >= p.n) {
#pragma unroll
          for (int qs = 0; qs < QS; ++qs) sacc[qs][v] = -INFINITY;
        }
      }
    }
    // ---- softmax bookkeeping per query sub-tile
    bf16x8 pf[QS][2];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; v += 2) mx = fmaxf(mx, fmaxf(sacc[qs][v], sacc[qs][v + 1]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (first) {
        m_ref[qs] = mx;
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[qs][v] -= mx;
      } else if (__builtin_amdgcn_ballot_w64(mx > ATT_RESCALE) != 0) {
        const float sh = fmaxf(mx, 0.f);
        const float alpha = __builtin_amdgcn_exp2f(-sh);
        m_ref[qs] += sh;
        l_run[qs] *= alpha;
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[qs][v] -= sh;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[t][qs][v] *= alpha;
      }
      float rs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(sacc[qs][v]);
        rs += e;
        pf[qs][v / 8][v % 8] = (__bf16)e;
      }
      l_run[qs] += rs;
    }
    // ---- O^T += V^T P^T   (both query sub-tiles share each V fragment)
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int s = 2 * ks + s2;   // 16-key step within the 64-key V^T row
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(buf + voff[t] + (((2 * s + hl) ^ vg[t]) * 16));
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) oacc[t][qs] = mfma32(a, pf[qs][s2], oacc[t][qs]);
      }
    }
  };
  auto tile = [&](int kt, const char* buf) __attribute__((always_inline)) {
    half_tile(kt, 0, buf);
    half_tile(kt, 1, buf);
  };

  // ring: wait for this wave's loads of tile kt (one later tile may stay in
  // flight), barrier, refill the slot freed by tile kt-1 with tile kt+2, consume kt
  issue(0, ring);
  if (KT > 1) issue(1, ring + STAGE);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) {
      att_wait_vmcnt<NI>();
    } else {
      att_wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (kt + 2 < KT) issue(kt + 2, ring + ((kt + 2) % 3) * STAGE);
    tile(kt, ring + (kt % 3) * STAGE);
  }

#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const float inv = 1.0f / (l_run[qs] + __shfl_xor(l_run[qs], 32, 64));
    const int qrow = q0 + qs * 32 + lq;
    if (qrow < p.n) {
      uint16_t* op = p.o + (size_t)qrow * p.heads * HD + head * HD;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = t * 32 + 8 * g + 4 * hl;
          const f32x16& a = oacc[t][qs];
          const uint2 w = make_uint2(pack2bf(a[4 * g] * inv, a[4 * g + 1] * inv),
                                     pack2bf(a[4 * g + 2] * inv, a[4 * g + 3] * inv));
          *reinterpret_cast<uint2*>(op + dd) = w;
        }
    }
  }
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((a.n + ATT_BQ - 1) / ATT_BQ, a.heads);
  if (a.head_dim == 128) {
    attn_kernel<128><<<grid, ATT_WAVES * 64, 0, s>>>(a);
  } else if (a.head_dim == 96) {
    attn_kernel<96><<<grid, ATT_WAVES * 64, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace h3
