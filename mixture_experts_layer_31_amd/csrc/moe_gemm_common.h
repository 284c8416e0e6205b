// Building blocks shared by the MFMA GEMM kernels (bf16 and fp8): buffer
// resources, direct-to-LDS loads, swizzled LDS tiles, operand stagers, the
// pipelined main loop and the accumulator layout.  See moe_gemm.hip for the
// design notes.
#pragma once

#include "moe_common.h"

namespace moe {
namespace gemm {

constexpr int kBK = 64;  // contraction step (bf16 elements)

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define AS3(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int xcd = b & 7, local = b >> 3;
  const int q = G >> 3, r = G & 7;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Raw buffer resource over [base, base + bytes): loads at byte offsets >= bytes return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
  r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(int(bytes));
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at `voff` into LDS at lds_base + 16 * lane.
// Issued as inline asm so the compiler does not serialise on it; completion is
// awaited explicitly with wait_vmcnt before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(AS3(p)));
}

// Chunk swizzles (chunk = 16 bytes = 8 bf16).
__device__ __forceinline__ int swz_k(int row) { return (row >> 1) & 7; }
template <int R>
__device__ __forceinline__ int swz_t(int krow) {
  if constexpr (R >= 128) return (krow & 3) << 2;
  else return ((krow >> 1) & 1) << 2;
}

// ---------------------------------------------------------------------------
// Operand stagers.  Each knows, per lane, the byte offset (relative to its
// buffer resource, at k-step 0) of the 16-byte chunk that lane fetches for each
// of the wave's DMA instructions, and how far that offset moves per k-step.

// k-contiguous operand, R rows: row r of the tile is at rowoff(r) bytes.
template <int R, int WAVES>
struct KStager {
  static constexpr int NI = R / (8 * WAVES);  // DMA instructions per wave per k-step (1 KB each)
  i32x4 rsrc;
  int vb[NI];
  template <class RowOff>
  __device__ __forceinline__ void init(i32x4 r, RowOff rowoff, int wave, int lane) {
    rsrc = r;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = wave * NI + j;
      const int row = q * 8 + (lane >> 3);
      const int logical = (lane & 7) ^ swz_k(row);
      const int ro = rowoff(row);
      vb[j] = ro < 0 ? int(0x80000000u) : ro + logical * 16;
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds, int wave, int kt) const {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      dma16(rsrc, lds + uint32_t(wave * NI + j) * 1024u, vb[j] + kt * (kBK * 2));
  }
};

// k-outer operand, R output columns: k-row k of the tile is at k * ld_bytes,
// column c at c * 2 (relative to the resource base, which includes the tile's
// first column).
template <int R, int WAVES>
struct TStager {
  static constexpr int NI = R / (8 * WAVES);
  static constexpr int LPR = R / 8;      // lanes per k-row
  static constexpr int RPI = 64 / LPR;   // k-rows per DMA instruction
  i32x4 rsrc;
  int vb[NI];
  int step;  // bytes per k-step
  __device__ __forceinline__ void init(i32x4 r, int ld_bytes, int wave, int lane) {
    rsrc = r;
    step = ld_bytes * kBK;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = wave * NI + j;
      const int krow = q * RPI + lane / LPR;
      const int logical = (lane % LPR) ^ swz_t<R>(krow);
      vb[j] = krow * ld_bytes + logical * 16;
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds, int wave, int kt) const {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      dma16(rsrc, lds + uint32_t(wave * NI + j) * 1024u, vb[j] + kt * step);
  }
};

// Fragment reads (8 consecutive k of one row/column, k-step sub-block kk).
__device__ __forceinline__ bf16x8 frag_k(const char* tile, int row, int kk, int lane) {
  const int chunk = kk * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(tile + row * 128 + ((chunk ^ swz_k(row)) << 4));
}

template <int R>
__device__ __forceinline__ bf16x8 frag_t(const char* tile, int col0, int kk, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  i16x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int krow = kk * 16 + 8 * (g >> 1) + 4 * half + (s >> 2);
    const char* p = tile + krow * (2 * R) + (((col >> 3) ^ swz_t<R>(krow)) << 4) + (col & 7) * 2;
    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)AS3(p));
  }
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}

// The pipelined main loop: acc += A_tile * B_tile^T over ktiles k-steps.  The
// workgroup's WGM x WGN waves each own a (BM/WGM) x (BN/WGN) sub-tile.  The
// MFMA takes the B fragment as its first operand, so an accumulator register
// block holds C^T: lane l owns output row (l & 31) of a 32 x 32 block and four
// consecutive output columns per group of four registers (see acc_col).
template <int BM, int BN, int WGM, int WGN, int STAGES, bool A_T, bool B_T, class SA, class SB>
__device__ __forceinline__ void mainloop(char* smem, const SA& sa, const SB& sb, int ktiles,
                                         f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32], int wave,
                                         int lane) {
  constexpr int WM = BM / WGM, WN = BN / WGN, WMT = WM / 32, WNT = WN / 32;
  constexpr int A_BYTES = BM * kBK * 2, STAGE = (BM + BN) * kBK * 2;
  constexpr int NI = SA::NI + SB::NI;  // DMA instructions per wave per stage
  const int wm = wave / WGN, wn = wave % WGN;
  const uint32_t base = lds_addr(smem);

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < ktiles) {
      sa.issue(base + s * STAGE, wave, s);
      sb.issue(base + s * STAGE + A_BYTES, wave, s);
    }

  for (int kt = 0; kt < ktiles; ++kt) {
    // wait for this wave's loads of k-step kt (later stages may stay in flight)
    const int ahead = min(ktiles - 1 - kt, STAGES - 2);
    if constexpr (STAGES >= 4) {
      if (ahead >= 2) wait_vmcnt<2 * NI>();
      else if (ahead == 1) wait_vmcnt<NI>();
      else wait_vmcnt<0>();
    } else if constexpr (STAGES == 3) {
      if (ahead >= 1) wait_vmcnt<NI>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    const int kn = kt + STAGES - 1;
    if (kn < ktiles) {
      const int sn = kn % STAGES;
      sa.issue(base + sn * STAGE, wave, kn);
      sb.issue(base + sn * STAGE + A_BYTES, wave, kn);
    }
    const char* ta = smem + (kt % STAGES) * STAGE;
    const char* tb = ta + A_BYTES;
    // fragments of sub-step kk+1 are read while the MFMAs of sub-step kk run
    bf16x8 af[2][WMT], bfr[2][WNT];
    auto load = [&](int kk, bf16x8 (&a)[WMT], bf16x8 (&b)[WNT]) {
#pragma unroll
      for (int i = 0; i < WMT; ++i) {
        const int r0 = wm * WM + i * 32;
        if constexpr (A_T) a[i] = frag_t<BM>(ta, r0, kk, lane);
        else a[i] = frag_k(ta, r0 + (lane & 31), kk, lane);
      }
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        const int c0 = wn * WN + j * 32;
        if constexpr (B_T) b[j] = frag_t<BN>(tb, c0, kk, lane);
        else b[j] = frag_k(tb, c0 + (lane & 31), kk, lane);
      }
    };
    load(0, af[0], bfr[0]);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      if (kk + 1 < kBK / 16) load(kk + 1, af[(kk + 1) & 1], bfr[(kk + 1) & 1]);
#pragma unroll
      for (int i = 0; i < WMT; ++i)
#pragma unroll
        for (int j = 0; j < WNT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk & 1][j], af[kk & 1][i],
                                                              acc[i][j], 0, 0, 0);
    }
  }
}

// Column (within a 32x32 block) of accumulator register 4*g (the first of four
// consecutive columns); the row is lane & 31.
__device__ __forceinline__ int acc_col(int g, int lane) { return 8 * g + 4 * (lane >> 5); }

template <int A, int B>
__device__ __forceinline__ void zero(f32x16 (&acc)[A][B]) {
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2(uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16),
                    uint32_t(f2bf(c)) | (uint32_t(f2bf(d)) << 16));
}

__device__ __forceinline__ void unpack4(uint2 v, float (&f)[4]) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
}

// Tile shape of a GEMM kernel: BM x BN outputs per workgroup of WGM x WGN waves.
template <int BM_, int BN_, int WGM_, int WGN_, int STAGES_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, STAGES = STAGES_;
  static constexpr int WAVES = WGM * WGN, THREADS = 64 * WAVES;
  static constexpr int WM = BM / WGM, WN = BN / WGN, WMT = WM / 32, WNT = WN / 32;
  static constexpr int LDS = STAGES * (BM + BN) * kBK * 2;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32x32");
};

enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

struct EpiArgs {
  uint16_t* out;          // STORE: [rows, ldo]; SWIGLU: H [rows, 2F]; DSWIGLU: dH [rows, 2F]
  int ldo;
  uint16_t* out2;         // SWIGLU: A [rows, F]
  const uint16_t* hsave;  // DSWIGLU: H [rows, 2F]
  int F;
};

// Epilogue of a token-grouped GEMM.  Lane owns row (lane & 31) of each 32-row
// block and, per group g of four registers, four consecutive columns starting
// at acc_col(g).  grow0 is the tile's first row in the permuted buffers.
template <class TL, int EPI>
__device__ __forceinline__ void grouped_epilogue(const EpiArgs& p,
                                                 f32x16 (&acc)[TL::WMT][TL::WNT], size_t grow0,
                                                 int rows_valid, int nt, int wm, int wn, int lane) {
  constexpr int BN = TL::BN, WM = TL::WM, WN = TL::WN, WMT = TL::WMT, WNT = TL::WNT;
#pragma unroll
  for (int i = 0; i < WMT; ++i) {
    const int m = wm * WM + i * 32 + (lane & 31);
    if (m >= rows_valid) continue;
    const size_t row = grow0 + m;
    if constexpr (EPI == EPI_STORE) {
#pragma unroll
      for (int j = 0; j < WNT; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = nt * BN + wn * WN + j * 32 + acc_col(g, lane);
          const f32x16& a = acc[i][j];
          *reinterpret_cast<uint2*>(p.out + row * p.ldo + n) =
              pack4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
      const int F = p.F;
#pragma unroll
      for (int j = 0; j < WNT / 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = nt * (BN / 2) + wn * (WN / 2) + j * 32 + acc_col(g, lane);
          float gv[4], uv[4], av[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            gv[c] = acc[i][j][4 * g + c];
            uv[c] = acc[i][j + WNT / 2][4 * g + c];
            av[c] = gv[c] / (1.f + __expf(-gv[c])) * uv[c];
          }
          *reinterpret_cast<uint2*>(p.out + row * 2 * F + f) = pack4(gv[0], gv[1], gv[2], gv[3]);
          *reinterpret_cast<uint2*>(p.out + row * 2 * F + F + f) = pack4(uv[0], uv[1], uv[2], uv[3]);
          *reinterpret_cast<uint2*>(p.out2 + row * F + f) = pack4(av[0], av[1], av[2], av[3]);
        }
    } else {  // EPI_DSWIGLU: acc holds dA = (w dy) W2[e] for the tile's F-columns
      const int F = p.F;
#pragma unroll
      for (int j = 0; j < WNT; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = nt * BN + wn * WN + j * 32 + acc_col(g, lane);
          float gv[4], uv[4], dg[4], du[4];
          unpack4(*reinterpret_cast<const uint2*>(p.hsave + row * 2 * F + f), gv);
          unpack4(*reinterpret_cast<const uint2*>(p.hsave + row * 2 * F + F + f), uv);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float dA = acc[i][j][4 * g + c];
            const float sg = 1.f / (1.f + __expf(-gv[c]));
            dg[c] = dA * uv[c] * sg * (1.f + gv[c] * (1.f - sg));
            du[c] = dA * gv[c] * sg;
          }
          *reinterpret_cast<uint2*>(p.out + row * 2 * F + f) = pack4(dg[0], dg[1], dg[2], dg[3]);
          *reinterpret_cast<uint2*>(p.out + row * 2 * F + F + f) = pack4(du[0], du[1], du[2], du[3]);
        }
    }
  }
}

// Epilogue of a per-expert weight-gradient GEMM: dW[e] tile (mt, nt) of [M, N].
template <class TL, bool OUT_F32>
__device__ __forceinline__ void wgrad_epilogue(void* C, int M, int N, int e, int mt, int nt,
                                               f32x16 (&acc)[TL::WMT][TL::WNT], int wm, int wn,
                                               int lane) {
#pragma unroll
  for (int i = 0; i < TL::WMT; ++i) {
    const int m = mt * TL::BM + wm * TL::WM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TL::WNT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nt * TL::BN + wn * TL::WN + j * 32 + acc_col(g, lane);
        const size_t o = (size_t(e) * M + m) * N + n;
        const f32x16& a = acc[i][j];
        if constexpr (OUT_F32)
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(C) + o) =
              make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        else
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(C) + o) =
              pack4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
      }
  }
}

}  // namespace gemm
}  // namespace moe
