// bf16 MFMA GEMM for the four linear layers of the H3 block, with the
// element-wise work of each layer fused into its epilogue (gfx950).
//
//   C[M][n_out] = A[M][K] . B[n_out][K]^T       (A = activations, B = weights,
//                                                 both K-contiguous)
//
// bf16 weights (gemm_direct_kernel): 256 x 256 block tile (256 x 192 for the
// 96-wide heads of the small model), four wavefronts in 2 x 2, each owning a
// 128 x 128 (x 96) sub-tile of v_mfma_f32_32x32x16_bf16 accumulators.  Tiles
// move HBM/L2 -> LDS with global_load_lds_dwordx4 (no staging registers) in
// stages of BK = 64, so each row segment is one full 128-byte line (measured to
// stream at twice the rate of 64-byte segments).  The LDS ring holds five
// half-stage slots (an A or a B half of a stage each, 32 KB): while one stage
// is consumed, the next stage and half of the one after are in flight.  The
// loads of a stage are spread over the MFMA stream, one after every MFMA
// quarter of a k step: a burst stalls the issuing wave until the load path has
// taken it, and with one wave per SIMD nothing else feeds the matrix core.  The
// K loop is unrolled by the ring period (5) so every slot offset is a
// compile-time immediate: loads take a wave-uniform SGPR base plus a per-lane
// offset fixed for the whole loop, and fragment reads a per-lane base plus an
// immediate, which keeps address arithmetic out of the loop.  Chunk c of LDS
// row r is stored at position c ^ f(r), f(r) = (r ^ (r>>3)) & 7, measured free
// of LDS bank conflicts for the 16-byte fragment reads; the permutation is
// applied by choosing which global chunk each lane of a load fetches.  Fragment
// reads of the next 16-wide k step are scheduled behind the current step's
// first MFMA.
//
// W8A8, group-scaled (gemm_w8a8g_kernel): int8 MFMAs into int32 accumulators
// per group of K elements, folded into fp32 with the group's activation and
// weight scales; eight wavefronts of 32 x 128 tiles, two per SIMD.
//
// INT8 weights (gemm_w8_kernel): eight wavefronts of 64 x 128 tiles; A streams
// in by DMA, int8 codes go through registers, where they are dequantised to
// bf16(q * s) (one bf16 scale per 32 K elements) on their way into a
// double-buffered LDS stage, interleaved with the MFMAs of the stage before.
//
// Block ids are remapped with the XCD in mind (blocks are dealt round-robin to
// the 8 XCDs): the 32 tiles an XCD runs at once are 8 row tiles x 4 column
// tiles (4 x 8 when K >= 7168), so each stage's A and B slices are shared in
// that XCD's L2; and over whole groups of 8 x that many row tiles the eight
// XCDs take one share each and walk the column tiles in step, so a weight
// panel comes from HBM once and the other seven XCDs find it in the shared
// Infinity Cache.
//
// MFMA 32x32 accumulator layout: lane l, register v holds
//   row = 8*(v/4) + 4*(l/32) + (v%4),   col = l%32.
//
// Epilogues (page titles and sections):
//  EPI_RESID  x[r][c] += gate[tag_r][c] * (acc + bias[c])  -- residual gate of
//             the attention and MLP branches (minimax-h3-mlx README, "AdaLN:
//             measure, do not reason": x + gate * f(x)).  fp32 in place.
//  EPI_SWIGLU weights rows are [gate; value]; each wave's N range is half gate
//             rows and half the matching value rows, so silu(g)*v is formed in
//             registers (staged through LDS for 16-byte row stores) and only
//             the F-wide activation is written
//             (minimax-h3-mlx README, "Validation": fc2(silu(gate) * value);
//             H3-metal digest, "Metal 4 and TensorOps paths": paired gate/up
//             tiles apply SwiGLU before writing).
//  EPI_STORE  x[r][c] = acc + bias[c], fp32 (the text condition projection
//             into the stream's text rows, and the narrow output heads).
//  EPI_QKV    each wave's N range is exactly one head_dim section of the
//             per-head interleaved [q|k|v] projection; q and k get RMSNorm
//             over the section (half-wave butterfly), the gain, and the rotary
//             turn (pair partner is the neighbouring lane), q is pre-scaled by
//             log2(e)/sqrt(d) for the exp2 softmax, and the results are
//             scattered head-major: q, k [H][n_pad][d], v transposed
//             [H][d][n_pad] (H3-metal digest, "Checkpoint layout and media
//             pipeline" and "Metal 4 and TensorOps paths": fused
//             QK-normalisation/RoPE, Q/K/V routed straight to head-major
//             attention inputs).
#include <type_traits>

#include "h3_device.h"
#include "launch.h"

namespace h3 {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait until at most N vector-memory operations of this wave are outstanding.
// Written as asm with a memory clobber so no LDS access moves across it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

struct TileCoord {
  int tm, tn;
};

template <int EPI, int BM, int BN>
__device__ __forceinline__ TileCoord tile_coord(const GemmArgs& p) {
  const int tiles_m = (EPI == EPI_QKV) ? p.n_pad / BM : (p.M + BM - 1) / BM;
  const int tiles_n = (p.n_out + BN - 1) / BN;
  // row tiles per XCD group: 8 x 4 tiles run at once, or 4 x 8 for long K, whose
  // activation panels are too large to stay cached across passes over the columns
  const int GROUP_M = p.K >= 7168 ? 4 : 8;
  const int raw = blockIdx.x;
  const int xcd = raw % 8;
  // full super-groups of 8 x GROUP_M row tiles: XCD x takes GROUP_M of them and
  // all XCDs walk the column tiles in step (shared weight panels)
  const int sgt = 8 * GROUP_M * tiles_n;
  const int full = tiles_m / (8 * GROUP_M);
  if (raw < full * sgt) {
    const int local = raw / 8;
    const int sg = local / (GROUP_M * tiles_n), l = local % (GROUP_M * tiles_n);
    return {sg * 8 * GROUP_M + xcd * GROUP_M + l % GROUP_M, l / GROUP_M};
  }
  // the remaining row tiles: contiguous runs per XCD, grouped GROUP_M rows at a time
  const int rm0 = full * 8 * GROUP_M, rtm = tiles_m - rm0;
  const int rraw = raw - full * sgt;
  const int total = rtm * tiles_n;
  const int per = total / 8, rem = total % 8;
  const int local = rraw / 8;
  const int pid = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int in_group = GROUP_M * tiles_n;
  const int first_m = (pid / in_group) * GROUP_M;
  const int gsz = min(rtm - first_m, GROUP_M);
  return {rm0 + first_m + (pid % in_group) % gsz, (pid % in_group) / gsz};
}

// Weight row feeding tile column r of tile tn (SwiGLU pairs gate and value rows per wave).
template <int EPI, int BN, int TN>
__device__ __forceinline__ int weight_row(const GemmArgs& p, int tn, int r) {
  if (EPI == EPI_SWIGLU) {
    const int w = r / TN, cc = r % TN, half = TN / 2;
    const int base = tn * (BN / 2) + w * half;
    return cc < half ? base + cc : p.ffn + base + cc - half;
  }
  return min(tn * BN + r, p.n_out - 1);
}

// Per-element QKV epilogue for head sections other than 128 wide (the
// 96-wide sections of the small model); the wider sections and the other
// epilogues go through LDS (below).
template <int BM, int BN, int WM, int WN, int EPI, int SEC, int FM, int FN>
__device__ __forceinline__ void epilogue(const GemmArgs& p, f32x16 (&acc)[FM][FN], int m0, int n0,
                                         int tn, int wm, int wn, int lane, const int* s_tag) {
  static_assert(EPI == EPI_QKV, "only the QKV sections that the LDS path does not take come here");
  constexpr int TM = BM / WM, TN = BN / WN;
  const int hl = lane >> 5;     // half-wave: rows 4..7 of each group of 8
  const int lc = lane & 31;     // column within a 32-wide MFMA tile
  const int row_base = m0 + wm * TM;
  (void)tn;
  (void)s_tag;
  const int sec = (n0 + wn * TN) / SEC;
  if (sec >= 3 * p.heads) return;
  const int kind = sec % 3, head = sec / 3;
  const uint16_t* gam = kind == 0 ? p.gq : p.gk;
  float bias_c[FN], gain_c[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = j * 32 + lc;
    bias_c[j] = p.bias ? bf2f(p.bias[sec * SEC + c]) : 0.f;
    gain_c[j] = (kind < 2 && gam) ? bf2f(gam[c]) : 1.f;
  }
  const float2* cs = reinterpret_cast<const float2*>(p.cs);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    float u[FN][16];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) u[j][v] = acc[i][j][v] + bias_c[j];
    if (kind < 2) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < FN; ++j) ss += u[j][v] * u[j][v];
        ss = half_sum(ss);
        const float r = 1.0f / sqrtf(ss / (float)SEC + p.qk_eps);
        const int row = row_base + i * 32 + 8 * (v / 4) + 4 * hl + (v % 4);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float t = u[j][v] * r * gain_c[j];
          const float partner = __shfl_xor(t, 1, 64);
          const int c = j * 32 + lc;
          const float2 sc = cs[(size_t)row * (SEC / 2) + c / 2];
          float o = (c & 1) ? partner * sc.y + t * sc.x : t * sc.x - partner * sc.y;
          if (kind == 0) o *= p.q_scale;
          u[j][v] = o;
        }
      }
    }
    uint16_t* dst = kind == 0 ? p.q : p.k;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = row_base + i * 32 + 8 * (v / 4) + 4 * hl + (v % 4);
      const bool valid = row < p.M;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int c = j * 32 + lc;
        const uint16_t val = valid ? f2bf(u[j][v]) : (uint16_t)0;
        if (kind < 2) {
          dst[((size_t)head * p.n_pad + row) * SEC + c] = val;
        } else {
          p.vt[((size_t)head * SEC + c) * p.n_pad + row] = val;
        }
      }
    }
  }
}

// Gated residual through LDS: each wavefront stages one 32-row slab of its
// accumulator tile at a time (fp32, padded rows), then reads it back as
// float4 along rows, so x is read and written in 16-byte coalesced pieces,
// the gate in 8-byte pieces, and the bias is loaded once per lane.  Without
// GATED the same path stores acc + bias (EPI_STORE).
constexpr int RSTRIDE = 136;   // floats per staged row (128 + 8 of padding)

template <bool GATED, int TM, int TN, int FM, int FN>
__device__ __forceinline__ void resid_epilogue_lds(const GemmArgs& p, f32x16 (&acc)[FM][FN],
                                                   int row0, int col0, int lane, float* stage,
                                                   const int* s_tag) {
  static_assert(TN == 128 || TN == 96 || TN == 64, "a half-wave's float4s cover one staged row");
  const int hl = lane >> 5, lc = lane & 31;
  const int gcol = col0 + 4 * lc;
  // n_out % 4 == 0, so a float4 is all in or all out; lanes past TN/4 idle
  const bool col_ok = 4 * lc < TN && gcol < p.n_out;
  float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p.bias && col_ok) {
    const u16x4 bb = *reinterpret_cast<const u16x4*>(p.bias + gcol);
    b4 = make_float4(bf2f(bb[0]), bf2f(bb[1]), bf2f(bb[2]), bf2f(bb[3]));
  }
  // 32 rows at a time: issue every gate and x load of the 32 rows, stage the
  // accumulators while they are in flight, then combine and store, so the
  // chunk waits for memory once rather than once per row (the stores could
  // alias the loads otherwise)
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    float4 xv[16];
    u16x4 gv[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int r = 2 * it + hl;
      const int row = row0 + i * 32 + r;
      if (GATED && row < p.M && col_ok) {
        const int t = s_tag[i * 32 + r];
        gv[it] = *reinterpret_cast<const u16x4*>(p.gate_tab + (size_t)t * p.tag_stride + gcol);
        xv[it] = *reinterpret_cast<const float4*>(p.x + (size_t)row * p.ldx + gcol);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        stage[(8 * (v / 4) + 4 * hl + (v % 4)) * RSTRIDE + j * 32 + lc] = acc[i][j][v];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int r = 2 * it + hl;
      const int row = row0 + i * 32 + r;
      const float4 a = *reinterpret_cast<const float4*>(stage + r * RSTRIDE + 4 * lc);
      if (row < p.M && col_ok) {
        float4 x;
        if constexpr (GATED) {
          x = xv[it];
          const u16x4 g = gv[it];
          x.x += bf2f(g[0]) * (a.x + b4.x);
          x.y += bf2f(g[1]) * (a.y + b4.y);
          x.z += bf2f(g[2]) * (a.z + b4.z);
          x.w += bf2f(g[3]) * (a.w + b4.w);
        } else {
          x = make_float4(a.x + b4.x, a.y + b4.y, a.z + b4.z, a.w + b4.w);
        }
        *reinterpret_cast<float4*>(p.x + (size_t)row * p.ldx + gcol) = x;
      }
    }
  }
}

// SwiGLU through LDS: a wavefront's N range is TN/2 gate columns and the
// matching TN/2 value columns; a = silu(g) * u is formed in registers, staged
// 32 rows at a time as fp32, and read back 8 values per lane along rows, so
// each row's TN/2 bf16 outputs (one 128-byte line for TN = 128) go out as
// 16-byte stores by 8 lanes.
constexpr int SSTRIDE = 68;   // floats per staged row (64 + 4 of padding)

template <int TM, int TN, int FM, int FN>
__device__ __forceinline__ void swiglu_epilogue_lds(const GemmArgs& p, f32x16 (&acc)[FM][FN],
                                                    int row0, int oc0, int lane, float* stage) {
  static_assert(TN == 128, "a wavefront writes 64 output columns per row");
  constexpr int H = FN / 2;
  const int hl = lane >> 5, lc = lane & 31;
  float bg[H], bv[H];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    bg[j] = p.bias ? bf2f(p.bias[oc0 + j * 32 + lc]) : 0.f;
    bv[j] = p.bias ? bf2f(p.bias[p.ffn + oc0 + j * 32 + lc]) : 0.f;
  }
  const int rr = lane >> 3, cc = 8 * (lane & 7);   // read-back: row rr (+8q), columns cc..cc+7
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < H; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float g = acc[i][j][v] + bg[j];
        const float u = acc[i][j + H][v] + bv[j];
        // silu(g) = g * 1/(1 + e^-g) with the hardware reciprocal (~1 ulp,
        // far below the bf16 rounding of the result); e^-g = inf gives 0
        stage[(8 * (v / 4) + 4 * hl + (v % 4)) * SSTRIDE + j * 32 + lc] =
            g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
      }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 8 * q + rr;
      const int row = row0 + i * 32 + r;
      const float4 a0 = *reinterpret_cast<const float4*>(stage + r * SSTRIDE + cc);
      const float4 a1 = *reinterpret_cast<const float4*>(stage + r * SSTRIDE + cc + 4);
      if (row < p.M)
        *reinterpret_cast<uint4*>(p.out + (size_t)row * p.ffn + oc0 + cc) =
            make_uint4(pack2bf(a0.x, a0.y), pack2bf(a0.z, a0.w), pack2bf(a1.x, a1.y), pack2bf(a1.z, a1.w));
    }
  }
}

// QKV epilogue through LDS (head_dim 128): each wavefront owns one 128-wide
// section (q, k or v of one head) and stages it 32 rows at a time.
//  q, k: lanes (row = l % 32, half = l / 32) read 64 values of a row as float4,
//        the RMS needs one cross-half add, rotary pairs sit inside each float4,
//        and the bf16 row half (128 B) is written with 16-byte stores.
//  v:    each lane takes two columns and writes 32 consecutive keys of V^T
//        (64 B) with 16-byte stores.
constexpr int QSTRIDE = 136;   // floats per staged row

template <int TM, int FM, int FN>
__device__ __forceinline__ void qkv_epilogue_lds(const GemmArgs& p, f32x16 (&acc)[FM][FN],
                                                 int row0, int sec, int lane, float* stage) {
  static_assert(FN == 4, "one 128-wide head section per wavefront");
  const int kind = sec % 3, head = sec / 3;
  const int hl = lane >> 5, lc = lane & 31;
  float bias_c[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) bias_c[j] = p.bias ? bf2f(p.bias[sec * 128 + j * 32 + lc]) : 0.f;
  const uint16_t* gam = kind == 0 ? p.gq : p.gk;
  // the norm gain of this lane's 64 columns, loaded once (q and k sections)
  const int c0 = 64 * hl;
  u16x4 gv[16];
  if (kind < 2) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      gv[k] = gam ? *reinterpret_cast<const u16x4*>(gam + c0 + 4 * k) : u16x4{0x3f80, 0x3f80, 0x3f80, 0x3f80};
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        stage[(8 * (v / 4) + 4 * hl + (v % 4)) * QSTRIDE + j * 32 + lc] = acc[i][j][v] + bias_c[j];
    const int slab = row0 + i * 32;
    if (kind < 2) {
      const int r = lc;
      const int row = slab + r;
      const float* src = stage + r * QSTRIDE + c0;
      // every rotary (cos, sin) load of the row before the first store, so the
      // row waits for memory once (the stores could alias the loads otherwise)
      const float4* cs = reinterpret_cast<const float4*>(p.cs + (size_t)row * 128 + c0);
      float4 tv[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) tv[k] = cs[k];
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float4 u = *reinterpret_cast<const float4*>(src + 4 * k);
        ss += (u.x * u.x + u.y * u.y) + (u.z * u.z + u.w * u.w);
      }
      ss += __shfl_xor(ss, 32, 64);
      const float rn = 1.0f / sqrtf(ss / 128.0f + p.qk_eps);
      const float sc = kind == 0 ? rn * p.q_scale : rn;
      uint16_t* dst = (kind == 0 ? p.q : p.k) + ((size_t)head * p.n_pad + row) * 128 + c0;
      const bool valid = row < p.M;
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        uint32_t w[4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int c = 4 * (k + kk);
          const float4 u = *reinterpret_cast<const float4*>(src + c);
          const float4 t = tv[k + kk];   // (cos, sin) of the two pairs in u
          const u16x4 gg = gv[k + kk];
          const float g0 = bf2f(gg[0]), g1 = bf2f(gg[1]), g2 = bf2f(gg[2]), g3 = bf2f(gg[3]);
          const float a0 = u.x * g0, a1 = u.y * g1, b0 = u.z * g2, b1 = u.w * g3;
          const float o0 = (a0 * t.x - a1 * t.y) * sc, o1 = (a0 * t.y + a1 * t.x) * sc;
          const float o2 = (b0 * t.z - b1 * t.w) * sc, o3 = (b0 * t.w + b1 * t.z) * sc;
          w[2 * kk] = valid ? pack2bf(o0, o1) : 0u;
          w[2 * kk + 1] = valid ? pack2bf(o2, o3) : 0u;
        }
        *reinterpret_cast<uint4*>(dst + 4 * k) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
      uint16_t* vt = p.vt + (size_t)head * 128 * p.n_pad + slab;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c = lane + 64 * cc;
        uint32_t w[16];
#pragma unroll
        for (int r = 0; r < 32; r += 2) {
          const float x0 = slab + r < p.M ? stage[r * QSTRIDE + c] : 0.f;
          const float x1 = slab + r + 1 < p.M ? stage[(r + 1) * QSTRIDE + c] : 0.f;
          w[r / 2] = pack2bf(x0, x1);
        }
        uint4* d = reinterpret_cast<uint4*>(vt + (size_t)c * p.n_pad);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) d[q4] = make_uint4(w[4 * q4], w[4 * q4 + 1], w[4 * q4 + 2], w[4 * q4 + 3]);
      }
    }
  }
}

// ============================================================ bf16: direct-to-LDS
constexpr int DBK = 64;          // K elements per stage
constexpr int DROW = DBK * 2;    // bytes per LDS row: one full 128-byte line per row
constexpr int HSLOT = 32768;     // one half stage (256 rows of A, or of B)
constexpr int NSLOT = 5;         // ring of half-stage slots

// Chunk c of row r sits at position c ^ f(r); measured free of LDS bank
// conflicts for the fragment reads (row lane%32 of each 32-row tile, chunk
// 2*kk + lane/32).  Depends on bits 0..5 of r.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_t;
__device__ __forceinline__ bf16x8 lds_read16(uint32_t a) { return *(lds_bf16x8_t*)(size_t)a; }
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr_t)p; }

// 16 bytes per lane from sbase + voff (sbase wave-uniform, in SGPRs) straight
// into LDS at lds + 16*lane (M0).  Asm keeps the compiler's wait insertion from
// draining in-flight stages before LDS reads; completion is tracked with
// wait_vmcnt.  The compiler does not insert hazard wait states across an asm
// statement: on gfx9 a vector memory instruction reads its SGPR operands
// without waiting for a VALU instruction that writes them (five wait states
// are needed), so sbase must come from SALU arithmetic (kernel arguments,
// offsets), never from a v_readfirstlane just before the call.
__device__ __forceinline__ void dma16s(uint32_t voff, const char* sbase, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_from<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_from<0, N>(f);
}

// lowest weight row a tile reads (the per-lane offsets are relative to it)
template <int EPI, int BN>
__device__ __forceinline__ int weight_row_base(int tn) {
  return EPI == EPI_SWIGLU ? tn * (BN / 2) : tn * BN;
}

template <int V>
using ic = std::integral_constant<int, V>;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// W8A8 (I8): int32 accumulators from v_mfma_i32_32x32x32_i8 become
// float(acc) * s_a[row] * s_w[col] before the epilogue; every other step is the
// bf16 kernel's, since a 16-byte fragment holds 32 int8 values of K where it
// held 16 bf16 ones (same LDS layout, same loads, twice the K per stage).
template <int EPI, int BN, int TN, int FM, int FN>
__device__ __forceinline__ void scale_int_acc(const GemmArgs& p, f32x16 (&acc)[FM][FN], int tn,
                                              int row0, int wn, int lane) {
  const int hl = lane >> 5, lc = lane & 31;
  float sw[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) sw[j] = bf2f(p.Bs[weight_row<EPI, BN, TN>(p, tn, wn * TN + j * 32 + lc)]);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    f32x16 sr;
#pragma unroll
    for (int v = 0; v < 16; ++v) sr[v] = p.sa[min(row0 + i * 32 + 8 * (v / 4) + 4 * hl + (v % 4), p.M - 1)];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const f32x16 f = __builtin_convertvector(__builtin_bit_cast(i32x16, acc[i][j]), f32x16);
      acc[i][j] = f * sr * sw[j];
    }
  }
}

template <int EPI, int SEC, int BN, bool I8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_direct_kernel(GemmArgs p) {
  constexpr int BM = 256, WM = 2, WN = 2;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int NA = BM / 32, NB = BN / 32;   // 1 KB (8-row) loads per half stage per wave
  constexpr int NA2 = NA / 2, NB2 = NB / 2;
  constexpr int NM = FM * FN, Q = NM / 4;
  static_assert(BM % 32 == 0 && BN % 32 == 0 && BN <= 256, "half-stage split");
  static_assert(NM % 4 == 0, "MFMA quarters");
  static_assert(EPI != EPI_QKV || TN == SEC, "QKV wave tile must be one head section");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU needs paired gate/value tiles");

  __shared__ __attribute__((aligned(1024))) char ring[NSLOT * HSLOT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const TileCoord tc = tile_coord<EPI, BM, BN>(p);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int K = p.K;
  const uint32_t rowb = (uint32_t)K * (I8 ? 1 : 2);

  // Loads: wave-uniform tile bases (SGPRs) advanced 128 B per stage, plus
  // per-lane 32-bit offsets fixed for the whole K loop.  Load s of a half
  // covers rows 8*(wave + 4s) .. +7; lane l fills row 8*(wave + 4s) + l/8,
  // position l%8, which holds global chunk (l%8) ^ f(row).
  const char* baseA = reinterpret_cast<const char*>(p.A) + (size_t)m0 * rowb;
  const int b0 = weight_row_base<EPI, BN>(tc.tn);
  const char* baseB = reinterpret_cast<const char*>(p.B) + (size_t)b0 * rowb;
  uint32_t voA[NA], voB[NB];
#pragma unroll
  for (int s = 0; s < NA; ++s) {
    const int r = 8 * (wave + 4 * s) + lane / 8;
    voA[s] = (uint32_t)(min(m0 + r, p.M - 1) - m0) * rowb + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
  }
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    const int r = 8 * (wave + 4 * s) + lane / 8;
    voB[s] = (uint32_t)(weight_row<EPI, BN, TN>(p, tc.tn, r) - b0) * rowb + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
  }
  const uint32_t ring0 = lds_addr(ring);
  // this wave's part of a slot; re-defined (empty asm) at each step so the
  // per-load M0 values are formed next to their loads rather than hoisted
  uint32_t mw = __builtin_amdgcn_readfirstlane(ring0 + wave * 1024);
  // loads [lo, hi) of the A (B) half of stage ks into slot S
  auto dmaA = [&](auto S_, int ks, int lo, int hi) __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value;
    const char* sb = baseA + (size_t)ks * (DBK * 2);
#pragma unroll
    for (int s = lo; s < hi; ++s) dma16s(voA[s], sb, mw + S * HSLOT + s * 4096);
  };
  auto dmaB = [&](auto S_, int ks, int lo, int hi) __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value;
    const char* sb = baseB + (size_t)ks * (DBK * 2);
#pragma unroll
    for (int s = lo; s < hi; ++s) dma16s(voB[s], sb, mw + S * HSLOT + s * 4096);
  };

  // Fragment reads: row lane%32 of each 32-row tile, chunk 2*kk + lane/32 at
  // its swizzled position (bit 5 of the row, the tile parity, enters the
  // swizzle).  Per-lane bases for three 64 KB windows of the ring, so every
  // read is base + immediate.
  const int fr = lane & 31, hl = lane >> 5;
  uint32_t rA[3][2][4], rB[3][2][4];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t xa = fr * DROW + (((2 * kk + hl) ^ swz(fr + 32 * par)) * 16);
      const int pb = ((wn * TN) / 32 + par) & 1;
      const uint32_t xb = fr * DROW + (((2 * kk + hl) ^ swz(fr + 32 * pb)) * 16);
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        rA[w][par][kk] = ring0 + w * 65536 + wm * TM * DROW + xa;
        rB[w][par][kk] = ring0 + w * 65536 + wn * TN * DROW + xb;
      }
    }
  auto read_frags = [&](auto SA_, auto SB_, int kk, bf16x8 (&fa)[FM], bf16x8 (&fb)[FN]) __attribute__((always_inline)) {
    constexpr int SA = decltype(SA_)::value, SB = decltype(SB_)::value;
    constexpr int WA = SA * HSLOT / 65536, WB = SB * HSLOT / 65536;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = lds_read16(rA[WA][i & 1][kk] + (SA * HSLOT - WA * 65536) + i * 32 * DROW);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = lds_read16(rB[WB][j & 1][kk] + (SB * HSLOT - WB * 65536) + j * 32 * DROW);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
  auto mfma_range = [&](const bf16x8 (&fa)[FM], const bf16x8 (&fb)[FN], int q0, int q1) __attribute__((always_inline)) {
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      f32x16& c = acc[q / FN][q % FN];
      if constexpr (I8) {
        c = __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                __builtin_bit_cast(i32x4, fa[q / FN]), __builtin_bit_cast(i32x4, fb[q % FN]),
                __builtin_bit_cast(i32x16, c), 0, 0, 0));
      } else {
        c = mfma32(fa[q / FN], fb[q % FN], c);
      }
    }
  };
  // One k step: the next k step's fragment reads go behind its first MFMA, and
  // the group's loads are spread one part per MFMA quarter (a burst of loads
  // stalls the issuing wave until the load path accepts them, and with one
  // wave per SIMD nothing else feeds the matrix core meanwhile).
  auto group = [&](const bf16x8 (&fa)[FM], const bf16x8 (&fb)[FN], auto&& reads, auto&& loads) __attribute__((always_inline)) {
    reads();
    mfma_range(fa, fb, 0, Q);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, Q - 1, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_barrier(0);
      loads(q);
      __builtin_amdgcn_sched_barrier(0);
      if (q < 3) mfma_range(fa, fb, (q + 1) * Q, (q + 2) * Q);
    }
  };
  auto part = [](int lo, int hi, int q) __attribute__((always_inline)) { return lo + ((hi - lo) * q) / 4; };

  bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  // Ring of five half-stage slots: the A half of stage s in slot 2s % 5, its B
  // half in (2s+1) % 5.  Iteration kt computes stage kt; its four k-step groups
  // issue, in order, the second half of stage kt+1's B loads, stage kt+2's A
  // half (two groups), and, after the barrier that frees stage kt's slots, the
  // first half of stage kt+2's B loads.  Before that barrier stage kt+1 must
  // have landed, while stage kt+2's A half may stay in flight.  In the steady
  // loop U = kt % 5 fixes every slot at compile time.
  auto step = [&](auto U_, int kt) __attribute__((always_inline)) {
    constexpr int U = decltype(U_)::value;
    constexpr int SA = (2 * U) % 5, SB = (2 * U + 1) % 5;
    constexpr int SA1 = (2 * U + 2) % 5, SB1 = (2 * U + 3) % 5;
    constexpr int SA2 = (2 * U + 4) % 5, SB2 = (2 * U + 5) % 5;
    asm volatile("" : "+s"(mw));
    group(fa0, fb0, [&]() __attribute__((always_inline)) { read_frags(ic<SA>{}, ic<SB>{}, 1, fa1, fb1); },
          [&](int q) __attribute__((always_inline)) { dmaB(ic<SB1>{}, kt + 1, part(NB2, NB, q), part(NB2, NB, q + 1)); });
    group(fa1, fb1, [&]() __attribute__((always_inline)) { read_frags(ic<SA>{}, ic<SB>{}, 2, fa0, fb0); },
          [&](int q) __attribute__((always_inline)) { dmaA(ic<SA2>{}, kt + 2, part(0, NA2, q), part(0, NA2, q + 1)); });
    group(fa0, fb0, [&]() __attribute__((always_inline)) { read_frags(ic<SA>{}, ic<SB>{}, 3, fa1, fb1); },
          [&](int q) __attribute__((always_inline)) { dmaA(ic<SA2>{}, kt + 2, part(NA2, NA, q), part(NA2, NA, q + 1)); });
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): stage kt fully read
    wait_vmcnt<NA>();
    __builtin_amdgcn_s_barrier();
    group(fa1, fb1, [&]() __attribute__((always_inline)) { read_frags(ic<SA1>{}, ic<SB1>{}, 0, fa0, fb0); },
          [&](int q) __attribute__((always_inline)) { dmaB(ic<SB2>{}, kt + 2, part(0, NB2, q), part(0, NB2, q + 1)); });
  };

  // the same step with slots from the runtime phase and loads only where the
  // stage exists (the last few stages of the K loop)
  const int KT = K / (I8 ? 2 * DBK : DBK);   // stages of 128 bytes per row
  auto step_rt = [&](int kt) __attribute__((always_inline)) {
    const uint32_t oa = (uint32_t)((2 * kt) % 5) * HSLOT, ob = (uint32_t)((2 * kt + 1) % 5) * HSLOT;
    const uint32_t oa1 = (uint32_t)((2 * kt + 2) % 5) * HSLOT, ob1 = (uint32_t)((2 * kt + 3) % 5) * HSLOT;
    const uint32_t oa2 = (uint32_t)((2 * kt + 4) % 5) * HSLOT, ob2 = (uint32_t)((2 * kt + 5) % 5) * HSLOT;
    const bool n1 = kt + 1 < KT, n2 = kt + 2 < KT;
    auto rd = [&](uint32_t xa_, uint32_t xb_, int kk, bf16x8 (&fa)[FM], bf16x8 (&fb)[FN]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = lds_read16(rA[0][i & 1][kk] + xa_ + i * 32 * DROW);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = lds_read16(rB[0][j & 1][kk] + xb_ + j * 32 * DROW);
    };
    group(fa0, fb0, [&]() __attribute__((always_inline)) { rd(oa, ob, 1, fa1, fb1); },
          [&](int q) __attribute__((always_inline)) {
            if (n1) {
              const char* sb = baseB + (size_t)(kt + 1) * (DBK * 2);
#pragma unroll
              for (int s = part(NB2, NB, q); s < part(NB2, NB, q + 1); ++s) dma16s(voB[s], sb, mw + ob1 + s * 4096);
            }
          });
    group(fa1, fb1, [&]() __attribute__((always_inline)) { rd(oa, ob, 2, fa0, fb0); },
          [&](int q) __attribute__((always_inline)) {
            if (n2) {
              const char* sb = baseA + (size_t)(kt + 2) * (DBK * 2);
#pragma unroll
              for (int s = part(0, NA2, q); s < part(0, NA2, q + 1); ++s) dma16s(voA[s], sb, mw + oa2 + s * 4096);
            }
          });
    group(fa0, fb0, [&]() __attribute__((always_inline)) { rd(oa, ob, 3, fa1, fb1); },
          [&](int q) __attribute__((always_inline)) {
            if (n2) {
              const char* sb = baseA + (size_t)(kt + 2) * (DBK * 2);
#pragma unroll
              for (int s = part(NA2, NA, q); s < part(NA2, NA, q + 1); ++s) dma16s(voA[s], sb, mw + oa2 + s * 4096);
            }
          });
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    if (n2) {
      wait_vmcnt<NA>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    group(fa1, fb1, [&]() __attribute__((always_inline)) { if (n1) rd(oa1, ob1, 0, fa0, fb0); },
          [&](int q) __attribute__((always_inline)) {
            if (n2) {
              const char* sb = baseB + (size_t)(kt + 2) * (DBK * 2);
#pragma unroll
              for (int s = part(0, NB2, q); s < part(0, NB2, q + 1); ++s) dma16s(voB[s], sb, mw + ob2 + s * 4096);
            }
          });
  };

  dmaA(ic<0>{}, 0, 0, NA);
  dmaB(ic<1>{}, 0, 0, NB);
  if (KT > 1) {
    dmaA(ic<2>{}, 1, 0, NA);
    dmaB(ic<3>{}, 1, 0, NB2);
    wait_vmcnt<NA + NB2>();
  } else {
    wait_vmcnt<0>();
  }
  __builtin_amdgcn_s_barrier();
  read_frags(ic<0>{}, ic<1>{}, 0, fa0, fb0);
  int kt = 0;
  for (; kt + 7 <= KT; kt += 5) {
    step(ic<0>{}, kt);
    step(ic<1>{}, kt + 1);
    step(ic<2>{}, kt + 2);
    step(ic<3>{}, kt + 3);
    step(ic<4>{}, kt + 4);
  }
  for (; kt < KT; ++kt) step_rt(kt);
  __syncthreads();
  if constexpr (I8) scale_int_acc<EPI, BN, TN, FM, FN>(p, acc, tc.tn, m0 + wm * TM, wn, lane);
  if constexpr (EPI == EPI_RESID) {
    // the tile's row tags go to LDS past the four staging areas (the ring is free now)
    int* s_tag = reinterpret_cast<int*>(ring + 4 * 32 * RSTRIDE * sizeof(float));
    s_tag[tid] = p.tag[min(m0 + tid, p.M - 1)];
    __syncthreads();
    resid_epilogue_lds<true, TM, TN, FM, FN>(p, acc, m0 + wm * TM, n0 + wn * TN, lane,
                                             reinterpret_cast<float*>(ring) + wave * 32 * RSTRIDE, s_tag + wm * TM);
  } else if constexpr (EPI == EPI_STORE) {
    resid_epilogue_lds<false, TM, TN, FM, FN>(p, acc, m0 + wm * TM, n0 + wn * TN, lane,
                                              reinterpret_cast<float*>(ring) + wave * 32 * RSTRIDE, nullptr);
  } else if constexpr (EPI == EPI_QKV && SEC == 128) {
    const int sec = (n0 + wn * TN) / SEC;
    if (sec < 3 * p.heads)
      qkv_epilogue_lds<TM, FM, FN>(p, acc, m0 + wm * TM, sec, lane,
                                   reinterpret_cast<float*>(ring) + wave * 32 * QSTRIDE);
  } else if constexpr (EPI == EPI_SWIGLU && TN == 128) {
    swiglu_epilogue_lds<TM, TN, FM, FN>(p, acc, m0 + wm * TM, tc.tn * (BN / 2) + wn * (TN / 2), lane,
                                        reinterpret_cast<float*>(ring) + wave * 32 * SSTRIDE);
  } else {
    epilogue<BM, BN, WM, WN, EPI, SEC>(p, acc, m0, n0, tc.tn, wm, wn, lane, nullptr);
  }
}

// ============================================================ INT8: dequant into LDS
// Weights are int8 codes q with one bf16 scale s per 32 K elements; the MFMA
// operand is W = bf16(q*s) (q*s is exact in fp32, rounded to nearest even).
// Eight wavefronts, 4 x 2 of 64 x 128 (x 96) tiles, two waves per SIMD, and a
// two-buffer LDS pipeline with BK = 64 stages.  While stage kt is consumed:
// A of stage kt+1 streams in by DMA (as in the bf16 kernel), the int8 codes of
// stage kt+1 (loaded one stage earlier) are dequantised and written to LDS,
// interleaved with the MFMAs, and the codes of stage kt+2 are loaded into the
// same registers right after, so they have a whole stage to arrive.  Each code is turned into bf16(q*s) with one byte-to-float conversion
// of q + 128 and one exact FMA, (q + 128)*s - 128*s, then rounded.  A full
// wait the compiler can see ends every stage, so its own wait insertion never
// counts the DMA loads it cannot see.
template <int EPI, int SEC, int BN>
__global__ __launch_bounds__(512) void gemm_w8_kernel(GemmArgs p) {
  constexpr int BM = 256, WM = 4, WN = 2, NT = 512;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int NA = BM / 8 / 8;                 // 1 KB (8-row) A loads per wave per stage
  constexpr int NBC = (BN * 4 + NT - 1) / NT;    // 16-code chunks per thread per stage
  constexpr int ABUF = 32768, BOFF = 65536;      // A of buffer b at b*ABUF, B at BOFF + b*ABUF
  static_assert(EPI != EPI_QKV || TN == SEC, "QKV wave tile must be one head section");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU needs paired gate/value tiles");

  // two LDS buffers during the K loop; the epilogue stages 32 rows per wave here
  constexpr int EPI_BYTES = 8 * 32 * (RSTRIDE > QSTRIDE ? RSTRIDE : QSTRIDE) * 4;
  __shared__ __attribute__((aligned(1024))) char sm[4 * ABUF > EPI_BYTES ? 4 * ABUF : EPI_BYTES];
  __shared__ int s_tag[EPI == EPI_RESID ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const TileCoord tc = tile_coord<EPI, BM, BN>(p);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  if (EPI == EPI_RESID) {
    for (int i = tid; i < BM; i += NT) s_tag[i] = p.tag[min(m0 + i, p.M - 1)];
  }
  const int K = p.K;
  const uint32_t rowb = (uint32_t)K * 2;
  const uint32_t sm0 = lds_addr(sm);

  // A by DMA: load s covers rows 8*(wave + 8s) .. +7; lane l fills row
  // 8*(wave + 8s) + l/8, position l%8 holding global chunk (l%8) ^ f(row)
  const char* baseA = reinterpret_cast<const char*>(p.A) + (size_t)m0 * rowb;
  uint32_t voA[NA];
#pragma unroll
  for (int s = 0; s < NA; ++s) {
    const int r = 8 * (wave + 8 * s) + lane / 8;
    voA[s] = (uint32_t)(min(m0 + r, p.M - 1) - m0) * rowb + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
  }
  const uint32_t mw = __builtin_amdgcn_readfirstlane(sm0 + wave * 1024);
  auto dmaA = [&](int ks, uint32_t boff) __attribute__((always_inline)) {
    const char* sb = baseA + (size_t)ks * (DBK * 2);
#pragma unroll
    for (int s = 0; s < NA; ++s) dma16s(voA[s], sb, mw + boff + s * 8192);
  };

  // B: chunk i of thread t is row r = t/4 + 128*i, codes k = 16*(t%4) .. +15 of
  // the stage, i.e. bf16 chunks 2c and 2c+1 (c = t%4) of that LDS row
  // wave-uniform bases of the tile's weight rows and scale rows (SGPRs), per-lane
  // 32-bit offsets
  const int b0 = weight_row_base<EPI, BN>(tc.tn);
  const int8_t* bbase = reinterpret_cast<const int8_t*>(p.B) + (size_t)b0 * K;
  const uint16_t* sbase = p.Bs + (size_t)b0 * (K / 32);
  uint32_t boffs[NBC], soffs[NBC], bdst0[NBC], bdst1[NBC];
  bool bval[NBC];
#pragma unroll
  for (int i = 0; i < NBC; ++i) {
    const int r = tid / 4 + (NT / 4) * i, c = tid & 3;
    bval[i] = (NT / 4) * NBC <= BN || r < BN;   // compile-time true when every row exists
    const int rr = min(r, BN - 1);
    const uint32_t brow = (uint32_t)(weight_row<EPI, BN, TN>(p, tc.tn, rr) - b0);
    boffs[i] = brow * (uint32_t)K + 16 * c;
    soffs[i] = brow * (uint32_t)(K / 32) + c / 2;
    bdst0[i] = sm0 + BOFF + rr * DROW + (((2 * c) ^ swz(rr)) * 16);
    bdst1[i] = sm0 + BOFF + rr * DROW + (((2 * c + 1) ^ swz(rr)) * 16);
  }
  // one register set: a stage's codes are dequantised before the next stage's
  // codes are loaded into the same registers
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) u32x4_t lds_u4_t;
  u32x4_t qv[NBC];
  uint32_t sv[NBC];
  auto ldB = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NBC; ++i)
      if (bval[i]) {
        qv[i] = *reinterpret_cast<const u32x4_t*>(bbase + boffs[i] + (size_t)ks * DBK);
        sv[i] = sbase[soffs[i] + ks * 2];
      }
  };
  auto deqB = [&](uint32_t boff) __attribute__((always_inline)) {
    // the codes count as produced here: nothing computed from them moves above
    // this point (in particular not into the previous stage, where their loads
    // are still in flight)
#pragma unroll
    for (int i = 0; i < NBC; ++i) asm volatile("" : "+v"(qv[i]), "+v"(sv[i]));
#pragma unroll
    for (int i = 0; i < NBC; ++i)
      if (bval[i]) {
        const float sc = __uint_as_float(sv[i] << 16), msc = -128.0f * sc;
        const uint32_t w4[4] = {qv[i][0] ^ 0x80808080u, qv[i][1] ^ 0x80808080u,
                                qv[i][2] ^ 0x80808080u, qv[i][3] ^ 0x80808080u};
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = w4[e / 2];
          const int sh = (e % 2) * 16;
          const float lo = __builtin_fmaf((float)((word >> sh) & 0xffu), sc, msc);
          const float hi = __builtin_fmaf((float)((word >> (sh + 8)) & 0xffu), sc, msc);
          o[e] = pack2bf(lo, hi);
        }
        *(lds_u4_t*)(size_t)(bdst0[i] + boff) = u32x4_t{o[0], o[1], o[2], o[3]};
        *(lds_u4_t*)(size_t)(bdst1[i] + boff) = u32x4_t{o[4], o[5], o[6], o[7]};
      }
  };

  // fragment reads: row lane%32 of each 32-row tile, chunk 2*kk + lane/32;
  // A of buffer b at b*ABUF, B at BOFF + b*ABUF (one base each, immediates)
  const int fr = lane & 31, hl = lane >> 5;
  uint32_t rA[2][4], rB[2][4];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      rA[par][kk] = sm0 + wm * TM * DROW + fr * DROW + (((2 * kk + hl) ^ swz(fr + 32 * par)) * 16);
      const int pb = ((wn * TN) / 32 + par) & 1;
      rB[par][kk] = sm0 + BOFF + wn * TN * DROW + fr * DROW + (((2 * kk + hl) ^ swz(fr + 32 * pb)) * 16);
    }
  auto read_frags = [&](auto B_, int kk, bf16x8 (&fa)[FM], bf16x8 (&fb)[FN]) __attribute__((always_inline)) {
    constexpr int b = decltype(B_)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = lds_read16(rA[i & 1][kk] + b * ABUF + i * 32 * DROW);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = lds_read16(rB[j & 1][kk] + b * ABUF + j * 32 * DROW);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
  auto mfmas = [&](const bf16x8 (&fa)[FM], const bf16x8 (&fb)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
  };
  // a full wait the compiler's own bookkeeping sees (it also covers the DMA)
  auto wait_all = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0 << 8)); };

  const int KT = K / DBK;
  bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  // stage kt in buffer b = kt & 1.  The loads of stages kt+1 and kt+2 are
  // clamped to the last stage: past the end they refill the idle buffer with
  // valid data that is never read, so every stage has the same shape.
  auto stage = [&](auto B_, int kt) __attribute__((always_inline)) {
    constexpr int b = decltype(B_)::value, nb = b ^ 1;
    deqB(nb * ABUF);
    ldB(min(kt + 2, KT - 1));
    dmaA(min(kt + 1, KT - 1), nb * ABUF);
    read_frags(B_, 1, fa1, fb1);
    mfmas(fa0, fb0);
    read_frags(B_, 2, fa0, fb0);
    mfmas(fa1, fb1);
    read_frags(B_, 3, fa1, fb1);
    mfmas(fa0, fb0);
    wait_all();
    __builtin_amdgcn_s_barrier();
    // past the last stage the reads hit the other buffer and go unused
    read_frags(ic<nb>{}, 0, fa0, fb0);
    mfmas(fa1, fb1);
  };

  ldB(0);
  dmaA(0, 0);
  wait_all();
  deqB(0);
  ldB(min(1, KT - 1));
  wait_all();
  __builtin_amdgcn_s_barrier();
  read_frags(ic<0>{}, 0, fa0, fb0);
  for (int kt = 0; kt < KT; kt += 2) {   // KT is even (K % 128 == 0, checked at launch)
    stage(ic<0>{}, kt);
    stage(ic<1>{}, kt + 1);
  }
  __syncthreads();
  if constexpr (EPI == EPI_RESID) {
    resid_epilogue_lds<true, TM, TN, FM, FN>(p, acc, m0 + wm * TM, n0 + wn * TN, lane,
                                             reinterpret_cast<float*>(sm) + wave * 32 * RSTRIDE, s_tag + wm * TM);
  } else if constexpr (EPI == EPI_QKV && SEC == 128) {
    const int sec = (n0 + wn * TN) / SEC;
    if (sec < 3 * p.heads)
      qkv_epilogue_lds<TM, FM, FN>(p, acc, m0 + wm * TM, sec, lane,
                                   reinterpret_cast<float*>(sm) + wave * 32 * QSTRIDE);
  } else if constexpr (EPI == EPI_SWIGLU && TN == 128) {
    swiglu_epilogue_lds<TM, TN, FM, FN>(p, acc, m0 + wm * TM, tc.tn * (BN / 2) + wn * (TN / 2), lane,
                                        reinterpret_cast<float*>(sm) + wave * 32 * SSTRIDE);
  } else {
    epilogue<BM, BN, WM, WN, EPI, SEC>(p, acc, m0, n0, tc.tn, wm, wn, lane, s_tag);
  }
}

// ============================================================ W8A8, group-scaled
// Group-scaled W8A8 (mlx-h3 README, "Generate": the trunk linears as
// group-scaled W8A8, one scale per group of G = 64, 256, 448 or 896 K elements
// on both operands):
//   y[r][c] = sum_g s_a[g][r] * s_w[g][c] * sum_{k in g} q_a[r][k] * q_w[c][k]
// Each group's integer sum is exact in int32 (|sum| <= 896 * 127^2 < 2^24, so
// also exact as fp32), then folded into fp32 accumulators at the group's end:
//   f[r][c] += float(i[r][c]) * s_w[c] * s_a[r].
// Both accumulator sets live through the K loop.  The fold is VALU work that
// depends on the group's last MFMAs, so two wavefronts share each SIMD: one's
// fold runs beside the other's MFMAs.  That caps a wave at 256 registers, so
// wave tiles are 32 x 128 (64 int32 + 64 fp32 accumulators): eight wavefronts
// stacked 8 x 1 on a 256 x 128 block tile (256 x 96 for the 96-wide head
// sections of the small model), each wave owning whole head sections as the
// QKV epilogue needs.  v_mfma_i32_32x32x32_i8 takes 32 K per step, so a
// 128-byte stage row holds 4 steps and every group ends on an even step.
// Stages (A 32 KB + B 16 KB) move by DMA into a 3-stage ring with the bf16
// kernel's swizzle; with each stage come the scales of the (at most two)
// groups it touches: s_a for the 256 rows (1 KB) and s_w for the tile's
// columns, both contiguous in their group-major layouts.  The first step of a
// group starts its int32 accumulators from zero (the MFMA's C operand).
template <int EPI, int SEC, int BN, int G>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_w8a8g_kernel(GemmArgs p) {
  constexpr int NW = 8;                           // wavefronts
  constexpr int BM = 256, WM = NW, WN = 1;
  constexpr int TM = BM / WM, TN = BN / WN;       // 32 x BN
  constexpr int FM = TM / 32, FN = TN / 32;       // 1 x (4 or 3)
  constexpr int SK = 128;                         // K (bytes) per stage row
  constexpr int ABYTES = BM * SK, BBYTES = BN * SK;
  constexpr int STAGE = ABYTES + BBYTES;
  constexpr int NST = 3;                          // ring of stages
  constexpr int NSC = 4;                          // ring of scale slots (one more than stages)
  constexpr int SCL = 4096;                       // per stage: s_a of 2 groups, then s_w of 2 groups
  constexpr int NRA = BM / 8, NRB = BN / 8;       // 8-row (1 KB) blocks of A and B
  constexpr int NA = (NRA + NW - 1) / NW, NB = (NRB + NW - 1) / NW;   // loads per wave per stage
  constexpr int PER = NA + NB + 1;                // DMA instructions per wave per stage
  static_assert(EPI != EPI_QKV || TN == SEC, "QKV wave tile must be one head section");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU needs paired gate/value tiles");
  static_assert(NST * STAGE + NSC * SCL <= 160 * 1024, "LDS");
  static_assert(NW * 32 * RSTRIDE * 4 + BM * 4 <= NST * STAGE + NSC * SCL, "epilogue staging");
  __shared__ __attribute__((aligned(1024))) char ring[NST * STAGE + NSC * SCL];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave;                            // WN == 1
  const TileCoord tc = tile_coord<EPI, BM, BN>(p);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  constexpr int GK = G / 32;                      // MFMA steps per group
  // stages per period: the shortest run of stages that holds whole groups
  // (lcm(SK, G) / SK), so within a period every group boundary, fold and
  // first step of a group sits at a fixed step
  constexpr int P = (G % SK == 0) ? G / SK : (SK % G == 0 ? 1 : 2 * G / SK);
  static_assert((P * SK) % G == 0 && (G % 64) == 0, "group layout");
  const int K = p.K;
  const int ng = K / G;                           // groups
  const int KT = K / SK;                          // stages (a multiple of P)
  const uint32_t rowb = (uint32_t)K;
  const uint32_t ring0 = lds_addr(ring);
  const uint32_t scl0 = ring0 + NST * STAGE;

  // A / B loads: load s of a wave fills 8-row block rb = wave + 8s (past the
  // last block a wave repeats an earlier block's load, so every wave issues
  // the same number); lane l fills row 8*rb + l/8, position l%8, which holds
  // global chunk (l%8) ^ f(row)
  const char* baseA = reinterpret_cast<const char*>(p.A) + (size_t)m0 * rowb;
  const int b0 = weight_row_base<EPI, BN>(tc.tn);
  const char* baseB = reinterpret_cast<const char*>(p.B) + (size_t)b0 * rowb;
  uint32_t voA[NA], voB[NB], ldA[NA], ldB[NB];
#pragma unroll
  for (int s = 0; s < NA; ++s) {
    const int rb = (wave + NW * s) % NRA;
    const int r = 8 * rb + lane / 8;
    voA[s] = (uint32_t)(min(m0 + r, p.M - 1) - m0) * rowb + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    ldA[s] = __builtin_amdgcn_readfirstlane(rb * 1024);
  }
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    const int rb = (wave + NW * s) % NRB;
    const int r = 8 * rb + lane / 8;
    voB[s] = (uint32_t)(weight_row<EPI, BN, TN>(p, tc.tn, r) - b0) * rowb + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    ldB[s] = __builtin_amdgcn_readfirstlane(ABYTES + rb * 1024);
  }
  // scale loads, one per wave per stage: wave w brings (w & 2 ? s_w : s_a) of
  // the stage's (w & 1 ? last : first) group (waves 4-7 repeat waves 0-3):
  // s_a for the 256 rows (16 B per lane), s_w for the BN columns (8 per lane;
  // lanes past them repeat lane 0's piece)
  // (the wave index through readfirstlane: the choices below are then
  // scalar, and the scale pointer and its LDS slot are formed by SALU
  // instructions in SGPRs)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool sa_wave = (wave_u & 2) == 0;
  const int sub_w = wave_u & 1;
  uint32_t vo_s;
  if (sa_wave) {
    vo_s = (uint32_t)(m0 + 4 * lane) * 4;
  } else {
    const int c = lane < BN / 8 ? 8 * lane : 0;
    vo_s = (uint32_t)weight_row<EPI, BN, TN>(p, tc.tn, c) * 2;
  }
  const int nw = EPI == EPI_SWIGLU ? 2 * p.ffn : p.n_out;   // weight rows (s_w row length)
  const char* sbase = sa_wave ? reinterpret_cast<const char*>(p.sa) : reinterpret_cast<const char*>(p.Bs);
  const size_t sstride = sa_wave ? (size_t)p.sa_ld * 4 : (size_t)nw * 2;   // bytes per group
  const uint32_t sm0 = __builtin_amdgcn_readfirstlane(scl0) + (sa_wave ? 0 : 2048) + sub_w * 1024;
  auto group_lo = [&](int kt) { return (kt * SK) / G; };
  auto group_hi = [&](int kt) { return min((kt * SK + SK - 1) / G, ng - 1); };

  auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(ring0 + (uint32_t)slot * STAGE);
    const int sslot = kt & (NSC - 1);
    const char* sa_ = baseA + (size_t)kt * SK;
    const char* sb_ = baseB + (size_t)kt * SK;
#pragma unroll
    for (int s = 0; s < NA; ++s) dma16s(voA[s], sa_, so + ldA[s]);
#pragma unroll
    for (int s = 0; s < NB; ++s) dma16s(voB[s], sb_, so + ldB[s]);
    const int g = sub_w ? group_hi(kt) : group_lo(kt);
    dma16s(vo_s, sbase + (size_t)g * sstride, sm0 + sslot * SCL);
  };

  // fragment reads: row lane%32 of each 32-row tile, chunk 2*kk + lane/32 at
  // its swizzled position; per-lane bases for the wave's A rows, the two B row
  // parities and the four steps of a stage, plus the stage's slot offset
  const int fr = lane & 31, hl = lane >> 5;
  uint32_t rA[FM][4], rB[2][4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * TM + 32 * i + fr;
      rA[i][kk] = ring0 + r * SK + (((2 * kk + hl) ^ swz(r)) * 16);
    }
#pragma unroll
    for (int par = 0; par < 2; ++par)
      rB[par][kk] = ring0 + ABYTES + fr * SK + (((2 * kk + hl) ^ swz(fr + 32 * par)) * 16);
  }
  auto read_frags = [&](uint32_t so, int kk, i32x4 (&fa)[FM], i32x4 (&fb)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = __builtin_bit_cast(i32x4, lds_read16(rA[i][kk] + so));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[j] = __builtin_bit_cast(i32x4, lds_read16(rB[j & 1][kk] + so + j * 32 * SK));
  };
  // the same from bases that already hold the stage's slot offset (one add
  // per base per stage; the tile offsets are immediates)
  struct Bases {
    uint32_t a[FM][4], b[2][4];
  };
  auto stage_bases = [&](uint32_t so) __attribute__((always_inline)) {
    Bases t;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int i = 0; i < FM; ++i) t.a[i][kk] = rA[i][kk] + so;
      t.b[0][kk] = rB[0][kk] + so;
      t.b[1][kk] = rB[1][kk] + so;
    }
    return t;
  };
  auto read_frags_b = [&](const Bases& t, int kk, i32x4 (&fa)[FM], i32x4 (&fb)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = __builtin_bit_cast(i32x4, lds_read16(t.a[i][kk]));
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = __builtin_bit_cast(i32x4, lds_read16(t.b[j & 1][kk] + j * 32 * SK));
  };

  i32x16 iacc[FM][FN];
  f32x16 facc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) facc[i][j] = f32x16{};
  const i32x16 zero = {};
  auto mfmas = [&](const i32x4 (&fa)[FM], const i32x4 (&fb)[FN], bool first) __attribute__((always_inline)) {
    if (first) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) iacc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], zero, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          iacc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], iacc[i][j], 0, 0, 0);
    }
  };
  // f += float(i) * s_w[col] * s_a[row] with the group's scales from the
  // stage's scale slot (sub = 0: the stage's first group, 1: its last)
  auto fold = [&](int sslot, int sub) __attribute__((always_inline)) {
    const float* sa_l = reinterpret_cast<const float*>(ring + NST * STAGE + sslot * SCL + sub * 1024);
    const uint16_t* sw_l = reinterpret_cast<const uint16_t*>(ring + NST * STAGE + sslot * SCL + 2048 + sub * 1024);
    float sw[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) sw[j] = bf2f(sw_l[j * 32 + fr]);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float sr[16];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 s4 = *reinterpret_cast<const float4*>(sa_l + wm * TM + i * 32 + 8 * t + 4 * hl);
        sr[4 * t] = s4.x;
        sr[4 * t + 1] = s4.y;
        sr[4 * t + 2] = s4.z;
        sr[4 * t + 3] = s4.w;
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          facc[i][j][v] = __builtin_fmaf((float)iacc[i][j][v] * sw[j], sr[v], facc[i][j][v]);
    }
  };

  // Three stages in flight.  The barrier that hands a stage over sits in the
  // last MFMA step of the stage before: once this wave's reads of that step
  // have landed and the next stage's DMA is complete, the barrier frees the
  // slot just read for the stage three ahead, and the next stage's first
  // fragments are read while the step's MFMAs run.  Scale slots are one more
  // than stages, so a fold after that barrier still finds its group's scales.
  // The K loop is unrolled over a period of P stages, so folds and group
  // starts are compile-time and the only branches in it hold no LDS reads
  // (the compiler's LDS waits then track the prefetch exactly).
  issue(0, 0);
  if (KT > 1) issue(1, 1);
  if (KT > 2) issue(2, 2);
  if (KT > 2) {
    wait_vmcnt<2 * PER>();
  } else if (KT > 1) {
    wait_vmcnt<PER>();
  } else {
    wait_vmcnt<0>();
  }
  __builtin_amdgcn_s_barrier();
  i32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  read_frags(0, 0, fa0, fb0);
  for (int kt0 = 0; kt0 < KT; kt0 += P) {
    static_for<P>([&](auto U_) __attribute__((always_inline)) {
      constexpr int U = decltype(U_)::value;
      const int kt = kt0 + U;
      uint32_t so = (uint32_t)(kt % NST) * STAGE;
      uint32_t so_next = (uint32_t)((kt + 1) % NST) * STAGE;
      int sslot = kt & (NSC - 1);
      // formed here, not hoisted to the top of the period (with two folds per
      // period the hoisted copies of later stages' offsets spill registers)
      asm volatile("" : "+s"(so), "+s"(so_next), "+s"(sslot));
      const Bases bs = stage_bases(so);
      static_for<4>([&](auto KK_) __attribute__((always_inline)) {
        constexpr int KK = decltype(KK_)::value;
        constexpr int KS = 4 * U + KK;                 // MFMA step within the period
        i32x4 (&fa)[FM] = (KK & 1) ? fa1 : fa0;
        i32x4 (&fb)[FN] = (KK & 1) ? fb1 : fb0;
        i32x4 (&ga)[FM] = (KK & 1) ? fa0 : fa1;
        i32x4 (&gb)[FN] = (KK & 1) ? fb0 : fb1;
        constexpr bool FOLD = (KS + 1) % GK == 0;   // the step ends a group
        if constexpr (KK < 3) {
          // a fold inside the stage reads the next fragments after it
          // (fewer registers live across the fold)
          if constexpr (!FOLD) read_frags_b(bs, KK + 1, ga, gb);
        } else {
          // the next stage (past the last one this reads a slot nobody
          // writes any more; the values are not used)
          if (kt + 2 < KT) {
            wait_vmcnt<PER>();
          } else {
            wait_vmcnt<0>();
          }
          __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): this stage fully read
          __builtin_amdgcn_s_barrier();
          if (kt + 3 < KT) issue(kt + 3, kt % NST);
          read_frags(so_next, 0, ga, gb);
        }
        mfmas(fa, fb, KS % GK == 0);
        if constexpr (FOLD) {
          // the group just finished: its scales sit in this stage's slot,
          // first (sub 0) if it is the stage's first group
          constexpr int GREL = KS / GK;                           // group within the period
          constexpr int GLO = (U * SK) / G;                       // the stage's first group
          // kept in place: hoisting its scale loads over the MFMAs costs registers
          __builtin_amdgcn_sched_barrier(0);
          fold(sslot, GREL == GLO ? 0 : 1);
          // the folded sums are marked as defined here: otherwise the compiler
          // sinks a fold inside a stage (groups of 64 or 448) below the next
          // group's MFMAs, keeping both int32 accumulator sets live (spills)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(facc[i][j]));
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (KK < 3) read_frags_b(bs, KK + 1, ga, gb);
        }
      });
    });
  }
  __syncthreads();
  if constexpr (EPI == EPI_RESID) {
    int* s_tag = reinterpret_cast<int*>(ring + NW * 32 * RSTRIDE * sizeof(float));
    if (tid < BM) s_tag[tid] = p.tag[min(m0 + tid, p.M - 1)];
    __syncthreads();
    resid_epilogue_lds<true, TM, TN, FM, FN>(p, facc, m0 + wm * TM, n0, lane,
                                             reinterpret_cast<float*>(ring) + wave * 32 * RSTRIDE, s_tag + wm * TM);
  } else if constexpr (EPI == EPI_QKV && SEC == 128) {
    const int sec = n0 / SEC;
    if (sec < 3 * p.heads)
      qkv_epilogue_lds<TM, FM, FN>(p, facc, m0 + wm * TM, sec, lane,
                                   reinterpret_cast<float*>(ring) + wave * 32 * QSTRIDE);
  } else if constexpr (EPI == EPI_SWIGLU && TN == 128) {
    swiglu_epilogue_lds<TM, TN, FM, FN>(p, facc, m0 + wm * TM, tc.tn * (BN / 2), lane,
                                        reinterpret_cast<float*>(ring) + wave * 32 * SSTRIDE);
  } else {
    epilogue<BM, BN, WM, WN, EPI, SEC>(p, facc, m0, n0, tc.tn, wm, 0, lane, nullptr);
  }
}

// ============================================================ INT8 weights, dequantised once
// bf16 weights W = RNE_bf16(q * s) from INT8 group-32 codes [rows][K] and bf16
// scales [rows][K/32] (the values the dequantising GEMM forms in LDS: q * s is
// exact in fp32, then rounded once).  The block forward uses it when its
// workspace holds a layer's bf16 weights: at a few row tiles and beyond, one
// pass over the weights costs less than dequantising them once per row tile.
// A chunk is 16 consecutive codes of a row; K % 32 == 0, so chunk c lies in
// scale group c / 2 of the row-major [rows][K/32] scales, and no row index is
// needed.  Each thread takes four chunks 256 apart (a block covers 1,024
// consecutive chunks, 16 KB of codes): four 16-byte code loads and four scale
// loads are in flight before the first conversion, then eight 16-byte stores.
constexpr int DQ_PER_THREAD = 4;

__global__ __launch_bounds__(256) void dequant_w8_kernel(const int8_t* __restrict__ q, const uint16_t* __restrict__ sc,
                                                         uint16_t* __restrict__ out, int64_t chunks) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int64_t c0 = (int64_t)blockIdx.x * (256 * DQ_PER_THREAD) + threadIdx.x;
  u32x4_t w[DQ_PER_THREAD];
  float sv[DQ_PER_THREAD];
#pragma unroll
  for (int u = 0; u < DQ_PER_THREAD; ++u) {
    const int64_t c = c0 + 256 * u;
    if (c < chunks) {
      w[u] = *reinterpret_cast<const u32x4_t*>(q + c * 16);
      sv[u] = bf2f(sc[c >> 1]);
    }
  }
#pragma unroll
  for (int u = 0; u < DQ_PER_THREAD; ++u) {
    const int64_t c = c0 + 256 * u;
    if (c >= chunks) break;
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t word = w[u][e / 2];
      const int sh = (e % 2) * 16;
      const float lo = (float)(int8_t)((word >> sh) & 0xffu) * sv[u];
      const float hi = (float)(int8_t)((word >> (sh + 8)) & 0xffu) * sv[u];
      o[e] = pack2bf(lo, hi);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + c * 16);
    dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
  }
}

hipError_t launch_dequant_w8(const DequantArgs& a, hipStream_t s) {
  if (a.K % 32 != 0 || a.rows <= 0) return hipErrorInvalidValue;
  const int64_t chunks = (int64_t)a.rows * (a.K / 16);
  const int64_t blocks = (chunks + 256 * DQ_PER_THREAD - 1) / (256 * DQ_PER_THREAD);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dequant_w8_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(a.q, a.s, a.out, chunks);
  return hipGetLastError();
}

// ============================================================ dispatch
template <int BM, int BN>
static dim3 grid_for(int epi, const GemmArgs& a) {
  const int tiles_m = epi == EPI_QKV ? a.n_pad / BM : (a.M + BM - 1) / BM;
  const int tiles_n = (a.n_out + BN - 1) / BN;
  return dim3(tiles_m * tiles_n);
}

template <int EPI, int SEC, int BN, bool I8 = false>
static hipError_t run_direct(const GemmArgs& a, hipStream_t s) {
  gemm_direct_kernel<EPI, SEC, BN, I8><<<grid_for<256, BN>(EPI, a), 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int EPI, int SEC, int BN>
static hipError_t run_w8a8g(const GemmArgs& a, hipStream_t s) {
  const dim3 grid = grid_for<256, BN>(EPI, a);
  // the K loop runs whole periods of lcm(128, group) elements
  if (a.K % 128 != 0 || a.K % a.group != 0) return hipErrorInvalidValue;
  switch (a.group) {
    case 64: gemm_w8a8g_kernel<EPI, SEC, BN, 64><<<grid, 512, 0, s>>>(a); break;
    case 256: gemm_w8a8g_kernel<EPI, SEC, BN, 256><<<grid, 512, 0, s>>>(a); break;
    case 448: gemm_w8a8g_kernel<EPI, SEC, BN, 448><<<grid, 512, 0, s>>>(a); break;
    case 896: gemm_w8a8g_kernel<EPI, SEC, BN, 896><<<grid, 512, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int EPI, int SEC, int BN>
static hipError_t run_w8(const GemmArgs& a, hipStream_t s) {
  gemm_w8_kernel<EPI, SEC, BN><<<grid_for<256, BN>(EPI, a), 512, 0, s>>>(a);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Residual and store GEMMs have the narrowest outputs (hidden, or a head's
// patch width): when 256-wide tiles leave the last wave of tiles mostly empty,
// or the output is narrower than a tile, 192- or 128-wide tiles balance better
// at a cost per MFMA (a quarter or a half fewer MFMAs per fragment read and per
// byte staged; measured ~5 % and ~25 % on the H3 residual GEMMs).  Cost
// model: waves of tiles x work per tile x that factor; returns the tile width.
// 128-wide tiles win only when a single wave of them covers the output (at
// H3 width up to 1,536 rows: 1.5x at 1,192 rows).
static int resid_tile_width(const GemmArgs& a, bool allow128) {
  const long tiles_m = (a.M + 255) / 256, cus = device_cus();
  auto waves = [&](long bn) { return (tiles_m * ((a.n_out + bn - 1) / bn) + cus - 1) / cus; };
  const long c256 = waves(256) * 256 * 100, c192 = waves(192) * 192 * 105, c128 = waves(128) * 128 * 125;
  if (allow128 && c128 < c192 && c128 < c256) return 128;
  return c192 < c256 ? 192 : 256;
}
static bool resid_prefers_192(const GemmArgs& a) { return resid_tile_width(a, false) == 192; }

// Rows of a gated-residual GEMM are independent, so one call may also run as
// two launches over disjoint row ranges: whole 256-row tiles [0, rows1) at
// width bn, the rest at 128-wide tiles.  With the same cost model per launch
// (plus a twentieth of a 256-wide tile for the second launch), this wins when
// the last wave of the wide tiles would be mostly empty and the remaining rows
// fill one wave of narrow tiles: at H3 width and 7,461 rows, 24 row tiles at
// 256 wide make two full waves (504 tiles) and the last 6 row tiles one wave
// of 252 narrow tiles, against three waves of 256-wide tiles in one launch.
struct ResidPlan {
  int bn;      // tile width of the first launch
  int rows1;   // rows of the first launch (M: no second launch)
};
static ResidPlan resid_plan(const GemmArgs& a) {
  const long tiles_m = (a.M + 255) / 256, cus = device_cus();
  auto cost = [&](long rt, long bn) {
    const long tiles = rt * ((a.n_out + bn - 1) / bn);
    return (tiles + cus - 1) / cus * bn * (bn == 256 ? 100 : bn == 192 ? 105 : 125);
  };
  ResidPlan best{resid_tile_width(a, true), a.M};
  long bc = cost(tiles_m, best.bn);
  for (int bn : {256, 192}) {
    for (long r = 1; r < tiles_m; ++r) {
      const long c = cost(r, bn) + cost(tiles_m - r, 128) + 256 * 100 / 20;
      if (c < bc) {
        bc = c;
        best = {bn, (int)(r * 256)};
      }
    }
  }
  return best;
}
// the call's rows [r0, M) as a call of their own
static GemmArgs resid_rows_from(const GemmArgs& a, int r0, bool int8_a) {
  GemmArgs b = a;
  b.A = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(a.A) +
                                          (size_t)r0 * a.K * (int8_a ? 1 : 2));
  b.x = a.x + (size_t)r0 * a.ldx;
  b.tag = a.tag + r0;
  if (int8_a) b.sa = a.sa + r0;   // one activation scale per row
  b.M = a.M - r0;
  return b;
}
// WF: 0 bf16 weights, 1 INT8 W8A16, 2 W8A8 with one scale per row
template <int WF>
static hipError_t run_resid_width(int bn, const GemmArgs& a, hipStream_t s) {
  if constexpr (WF == 1) {
    if (bn == 128) return run_w8<EPI_RESID, 0, 128>(a, s);
    if (bn == 192) return run_w8<EPI_RESID, 0, 192>(a, s);
    return run_w8<EPI_RESID, 0, 256>(a, s);
  } else {
    if (bn == 128) return run_direct<EPI_RESID, 0, 128, WF == 2>(a, s);
    if (bn == 192) return run_direct<EPI_RESID, 0, 192, WF == 2>(a, s);
    return run_direct<EPI_RESID, 0, 256, WF == 2>(a, s);
  }
}
template <int WF>
static hipError_t run_resid(const GemmArgs& a, hipStream_t s) {
  const ResidPlan pl = resid_plan(a);
  if (pl.rows1 >= a.M) return run_resid_width<WF>(pl.bn, a, s);
  GemmArgs first = a;
  first.M = pl.rows1;
  const hipError_t e = run_resid_width<WF>(pl.bn, first, s);
  if (e != hipSuccess) return e;
  return run_resid_width<WF>(128, resid_rows_from(a, pl.rows1, WF == 2), s);
}

hipError_t launch_gemm(int epi, int wfmt, const GemmArgs& a, hipStream_t s) {
  if (a.K % 64 != 0) return hipErrorInvalidValue;
  if (wfmt != 0 && a.K % 128 != 0) return hipErrorInvalidValue;   // INT8: 128-element stages
  if (wfmt == 2 && a.group > 0) {   // W8A8, one scale per group of K elements on both operands
    if (a.K % a.group != 0 || a.group % 64 != 0 || a.n_out % 32 != 0) return hipErrorInvalidValue;
    switch (epi) {
      case EPI_RESID: return run_w8a8g<EPI_RESID, 0, 128>(a, s);
      case EPI_SWIGLU: return run_w8a8g<EPI_SWIGLU, 0, 128>(a, s);
      case EPI_QKV:
        if (a.head_dim == 128) return run_w8a8g<EPI_QKV, 128, 128>(a, s);
        if (a.head_dim == 96) return run_w8a8g<EPI_QKV, 96, 96>(a, s);
    }
    return hipErrorInvalidValue;
  }
  if (wfmt == 2) {   // W8A8 with one scale per row (FC2's per-row form)
    switch (epi) {
      case EPI_RESID: return run_resid<2>(a, s);
      case EPI_SWIGLU: return run_direct<EPI_SWIGLU, 0, 256, true>(a, s);
      case EPI_QKV:
        if (a.head_dim == 128) return run_direct<EPI_QKV, 128, 256, true>(a, s);
        if (a.head_dim == 96) return run_direct<EPI_QKV, 96, 192, true>(a, s);
    }
    return hipErrorInvalidValue;
  }
  if (wfmt == 0) {
    switch (epi) {
      case EPI_RESID: return run_resid<0>(a, s);
      case EPI_STORE:
        if (resid_prefers_192(a)) return run_direct<EPI_STORE, 0, 192>(a, s);
        return run_direct<EPI_STORE, 0, 256>(a, s);
      case EPI_SWIGLU: return run_direct<EPI_SWIGLU, 0, 256>(a, s);
      case EPI_QKV:
        if (a.head_dim == 128) return run_direct<EPI_QKV, 128, 256>(a, s);
        if (a.head_dim == 96) return run_direct<EPI_QKV, 96, 192>(a, s);
    }
    return hipErrorInvalidValue;
  }
  switch (epi) {   // (EPI_STORE layers have bf16 weights only)
    case EPI_RESID: return run_resid<1>(a, s);
    case EPI_SWIGLU: return run_w8<EPI_SWIGLU, 0, 256>(a, s);
    case EPI_QKV:
      if (a.head_dim == 128) return run_w8<EPI_QKV, 128, 256>(a, s);
      if (a.head_dim == 96) return run_w8<EPI_QKV, 96, 192>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace h3
