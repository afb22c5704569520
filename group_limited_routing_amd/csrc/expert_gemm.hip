// Grouped expert GEMMs of the Beam MoE block on gfx950.
//
// Beam launch post ("Introducing Beam"), section "Mixture of Experts": each
// expert is a SwiGLU MLP with intermediate size 2560; section "Residual
// Stream": the SwiGLU product is computed in fp32. Expert e computes
//   h = silu(x W_gate[e]^T) * (x W_up[e]^T)      (gate/up pass, "mode 0")
//   y = rsf * w * (h W_down[e]^T)                 (down pass, "mode 1")
// for the rows the permutation sorted into expert e's contiguous range.
//
// Both passes walk a device-built list of M-tiles (expert, first row). A
// workgroup takes one M-tile and one block of output columns; the grid is
// sized from a T-based bound on the tile count and surplus workgroups exit at
// once, so the host never reads the counts.
//
// Two variants:
//  * stream (few rows per expert, decode): 16-row M-tiles; every wave owns
//    its own weight rows and streams them from HBM straight into MFMA
//    operands through a D-deep register ring, with no LDS and no barriers.
//    The 16 token rows come from L2.
//  * tiled (prefill): 128-row M-tiles; the A rows and 128 weight rows are
//    staged through XOR-swizzled LDS, double buffered, and 4 waves each
//    compute a 64 x 64 block.
// In the gate/up pass a wave always holds the gate and the up accumulators
// of the same output columns, so the SwiGLU epilogue is elementwise.
//
// Weights are bf16 (16x16x32 bf16 MFMA) or OCP E4M3 codes with one fp32
// scale per output row (16x16x128 fp8 MFMA). With fp8 weights the A operand
// is E4M3 too (x quantised per token, h per row); the scales are applied to
// the fp32 accumulators in the epilogue, and the gate/up pass writes h as
// bf16 (as with bf16 weights) and records each row's max |h| of the stored
// values for the per-row quantisation of the down pass's input.
#include "common.h"
#include "internal.h"


namespace beam {

// Per-type constants. One MFMA consumes KSTEP values of k; a lane's operand
// is OPB bytes of one row.
template <bool FP8>
struct WTraits;
template <>
struct WTraits<false> {
  using W = uint16_t;
  static constexpr int KSTEP = 32, OPB = 16;
};
template <>
struct WTraits<true> {
  using W = uint8_t;
  static constexpr int KSTEP = 128, OPB = 32;
};

// A 32-byte operand register (fp8) or a 16-byte one (bf16).
struct Op32 {
  u32x4 lo, hi;
};

__device__ __forceinline__ f32x4 mfma_op(const u32x4& a, const u32x4& b, f32x4 c) {
  return mfma_bf16(as_bf16x8(a), as_bf16x8(b), c);
}
__device__ __forceinline__ f32x4 mfma_op(const Op32& a, const Op32& b, f32x4 c) {
  i32x8 av, bv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    av[i] = (int)a.lo[i];
    av[4 + i] = (int)a.hi[i];
    bv[i] = (int)b.lo[i];
    bv[4 + i] = (int)b.hi[i];
  }
  return mfma_fp8(av, bv, c);
}

template <bool FP8>
using OpReg = typename std::conditional<FP8, Op32, u32x4>::type;

template <bool FP8>
__device__ __forceinline__ OpReg<FP8> load_op(const void* p) {
  if constexpr (FP8) {
    Op32 o;
    o.lo = ld16(p);
    o.hi = ld16((const uint8_t*)p + 16);
    return o;
  } else {
    return ld16(p);
  }
}

// A weight operand: read once per workgroup, so loaded non-temporally.
template <bool FP8>
__device__ __forceinline__ OpReg<FP8> load_w(const void* p) {
  if constexpr (FP8) {
    Op32 o;
    o.lo = ld16_nt(p);
    o.hi = ld16_nt((const uint8_t*)p + 16);
    return o;
  } else {
    return ld16_nt(p);
  }
}


// The A operand of a bf16 pass may be stored as fp32 (x in fp32); it is then
// rounded to bf16 (nearest even) on load. 8 values per lane.
template <typename AT>
struct ALoad16;
template <>
struct ALoad16<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = ld16(p); }
  __device__ __forceinline__ u32x4 bits() const { return v; }
  __device__ __forceinline__ void floats(float* f) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_bits_to_f32(v[i] & 0xffffu);
      f[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
    }
  }
};
template <>
struct ALoad16<float> {
  u32x4 v0, v1;
  __device__ __forceinline__ void load(const float* p) {
    v0 = ld16(p);
    v1 = ld16(p + 4);
  }
  __device__ __forceinline__ void floats(float* f) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(v0[i]);
      f[4 + i] = __uint_as_float(v1[i]);
    }
  }
  __device__ __forceinline__ u32x4 bits() const {
    u32x4 o;
    o[0] = pack_bf16x2(__uint_as_float(v0[0]), __uint_as_float(v0[1]));
    o[1] = pack_bf16x2(__uint_as_float(v0[2]), __uint_as_float(v0[3]));
    o[2] = pack_bf16x2(__uint_as_float(v1[0]), __uint_as_float(v1[1]));
    o[3] = pack_bf16x2(__uint_as_float(v1[2]), __uint_as_float(v1[3]));
    return o;
  }
};

struct TileInfo {
  int e, row0, rows;
};

__device__ __forceinline__ bool tile_info(const GemmArgs& p, int mt, int BM, TileInfo& ti) {
  if (mt >= p.meta[0]) return false;
  ti.e = p.tile_e[mt];
  ti.row0 = p.tile_r[mt];
  ti.rows = min(BM, p.offsets[ti.e + 1] - ti.row0);
  return true;
}

// Epilogue of one 16x16 accumulator pair / block. `row` is the tile-local
// row, `n` the output column; returns nothing, stores one value.
template <bool FP8>
__device__ __forceinline__ float gateup_value(const GemmArgs& p, const TileInfo& ti, int row, int n,
                                              float gacc, float uacc) {
  if constexpr (FP8) {
    const float xs = p.a_scale[p.stok[ti.row0 + row]];
    const float gv = gacc * xs * p.ws0[(size_t)ti.e * p.N + n];
    const float uv = uacc * xs * p.ws1[(size_t)ti.e * p.N + n];
    return silu_f32(gv) * uv;
  } else {
    return silu_f32(gacc) * uacc;
  }
}

template <bool FP8>
__device__ __forceinline__ float down_value(const GemmArgs& p, const TileInfo& ti, int row, int n,
                                            float acc) {
  if constexpr (FP8) {
    return acc * p.a_scale[ti.row0 + row] * p.ws0[(size_t)ti.e * p.N + n] * p.sw[ti.row0 + row];
  } else {
    return acc * p.sw[ti.row0 + row];
  }
}

// h is stored as bf16 (round to nearest even); returns the stored value,
// whose magnitude enters the row's max |h| on the quantised paths.
__device__ __forceinline__ float store_h(const GemmArgs& p, size_t off, float h) {
  const uint32_t b = f32_to_bf16_bits(h);
  ((uint16_t*)p.out)[off] = (uint16_t)b;
  return bf16_bits_to_f32(b);
}

// Row-wise max |h| over the 16 columns a lane group holds, then one atomicMax
// per row. |h| >= 0, so its float bits order like unsigned integers; the
// maximum does not depend on the order of the updates.
__device__ __forceinline__ void row_amax_update(uint32_t* hamax, int grow, float v, bool valid) {
  float m = fabsf(v);
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (valid && (threadIdx.x & 15) == 0) atomicMax(&hamax[grow], __float_as_uint(m));
}

// ---------------------------------------------------------------- stream variant
// FN = 16-row weight fragments per wave (mode 0: FN/2 gate + FN/2 up),
// D = depth of the register prefetch ring (in MFMA k-steps), MR = 16-row
// blocks of tokens per M-tile (1 or 2): each weight fragment streamed from
// HBM feeds MR matrix-core steps, so an expert with up to 16 MR rows reads
// its weights once.
template <int MODE, typename AT, bool FP8, bool PACKED, int FN, int D, int MR>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs p) {
  using WT = typename WTraits<FP8>::W;
  constexpr int KSTEP = WTraits<FP8>::KSTEP;
  constexpr int LANE_K = KSTEP / 4;  // k values per lane per step
  constexpr int HALF = FN / 2;
  constexpr int COLS_W = (MODE == 0) ? 16 * HALF : 16 * FN;  // output columns per wave
  constexpr int COLS = 4 * COLS_W;                           // per workgroup
  static_assert(MR == 1 || MR == 2, "one or two row blocks");
  const int ntn = p.N / COLS;
  const int mt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  TileInfo ti;
  if (!tile_info(p, mt, 16 * MR, ti)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N;

  // Padded rows (row >= rows) repeat the last real row; their results are not stored.
  const AT* arow[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int ar = min(16 * m + r, ti.rows - 1);
    arow[m] = (MODE == 0) ? (const AT*)p.a + (size_t)p.stok[ti.row0 + ar] * K + LANE_K * g
                          : (const AT*)p.a + (size_t)(ti.row0 + ar) * K + LANE_K * g;
  }
  const int ncol0 = nt * COLS + wave * COLS_W;
  const WT* brow[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    int n;
    const WT* W;
    if (MODE == 0) {
      n = ncol0 + (f % HALF) * 16 + r;
      W = (const WT*)(f < HALF ? p.w0 : p.w1);
    } else {
      n = ncol0 + f * 16 + r;
      W = (const WT*)p.w0;
    }
    if (PACKED)  // fragment block (n / 16, step) starts at ((n/16) * K/KSTEP + step) * 16*KSTEP
      brow[f] = W + (size_t)ti.e * N * K + (size_t)((n - r) >> 4) * 16 * K + lane * LANE_K;
    else
      brow[f] = W + ((size_t)ti.e * N + n) * K + LANE_K * g;
  }
  constexpr int BSTEP = PACKED ? 16 * KSTEP : KSTEP;  // elements between k-steps of a lane

  f32x4 acc[MR][FN];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int f = 0; f < FN; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = K / KSTEP;  // K is a multiple of 128: bf16 nks % 4 == 0, fp8 nks >= 1
  using OR = OpReg<FP8>;
  OR bq[D][FN];
  OR aq8[FP8 ? D : 1][MR];
  using AL16 = typename std::conditional<FP8, ALoad16<uint16_t>, ALoad16<AT>>::type;
  AL16 aq16[FP8 ? 1 : D][MR];
  auto load_step = [&](int d, int s) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if constexpr (FP8)
        aq8[d][m] = load_op<true>(arow[m] + (size_t)s * KSTEP);
      else
        aq16[d][m].load((const typename std::conditional<FP8, uint16_t, AT>::type*)arow[m] +
                        (size_t)s * KSTEP);
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) bq[d][f] = load_w<FP8>(brow[f] + (size_t)s * BSTEP);
  };
  auto consume = [&](int d) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      OR a;
      if constexpr (FP8)
        a = aq8[d][m];
      else
        a = aq16[d][m].bits();
#pragma unroll
      for (int f = 0; f < FN; ++f) acc[m][f] = mfma_op(a, bq[d][f], acc[m][f]);
    }
  };
  // Prologue without branches (a step past the end, possible only when
  // K < D * KSTEP, re-reads the last step and is never consumed).
#pragma unroll
  for (int d = 0; d < D; ++d) load_step(d, min(d, nks - 1));
  // Steady state without branches around the loads, so the compiler's wait
  // counts let each step wait only for its own (oldest) loads while the
  // next D-1 steps stay in flight.
  int s0 = 0;
  for (; s0 + 2 * D <= nks; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      consume(d);
      load_step(d, s0 + d + D);
    }
  }
  // Tail: at most 2D - 1 steps left, D of them already loaded.
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (s0 + d < nks) {
      consume(d);
      if (s0 + d + D < nks) load_step(d, s0 + d + D);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (s0 + D + d < nks) consume(d);

  // Lane (r, g) of row block m holds rows 16 m + 4 g .. + 3 of column r.
  if (MODE == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * m + 4 * g + i;
        const bool valid = row < ti.rows;
        float rowmax = 0.f;
#pragma unroll
        for (int f = 0; f < HALF; ++f) {
          const int n = ncol0 + f * 16 + r;
          if (valid) {
            const float h = gateup_value<FP8>(p, ti, row, n, acc[m][f][i], acc[m][f + HALF][i]);
            const float hs = store_h(p, (size_t)(ti.row0 + row) * N + n, h);
            rowmax = fmaxf(rowmax, fabsf(hs));
          }
        }
        if constexpr (FP8) row_amax_update(p.hamax, ti.row0 + row, rowmax, valid);
      }
    }
  } else {
    uint16_t* out = (uint16_t*)p.out;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * m + 4 * g + i;
        if (row < ti.rows) {
#pragma unroll
          for (int f = 0; f < FN; ++f) {
            const int n = ncol0 + f * 16 + r;
            out[(size_t)(ti.row0 + row) * N + n] =
                (uint16_t)f32_to_bf16_bits(down_value<FP8>(p, ti, row, n, acc[m][f][i]));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- MXFP4 stream variant
// Expert GEMMs with MXFP4 weights (packed: one 1 KB block per 16 rows x 128
// reduction steps, two E2M1 codes per byte; E8M0 block scales packed so that
// one 4-byte load gives a lane the scales of four consecutive steps). The
// token rows are E4M3 codes with a per-row fp32 scale (applied in the
// epilogue); each 16x16x128 MFMA takes the weight fragment as its second
// operand together with the lane's block scale. Same M-tiles, waves and
// register ring as the streaming bf16/fp8 variant.
template <int MODE, int FN, int D, int MR>
__global__ __launch_bounds__(256) void gemm_stream4_kernel(GemmArgs p) {
  constexpr int HALF = FN / 2;
  constexpr int COLS_W = (MODE == 0) ? 16 * HALF : 16 * FN;  // output columns per wave
  constexpr int COLS = 4 * COLS_W;                           // per workgroup
  static_assert(MR == 1 || MR == 2, "one or two row blocks");
  const int ntn = p.N / COLS;
  const int mt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  TileInfo ti;
  if (!tile_info(p, mt, 16 * MR, ti)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N;

  // Padded rows (r >= rows) repeat the last real row; their results are not stored.
  // With an fp4 second operand the instruction pairs codes 0-15 of weight
  // lane group g with activation lane group 2 (g % 2) and codes 16-31 with
  // group 2 (g % 2) + 1, in activation bytes 0-15 for g < 2 and 16-31 for
  // g >= 2 (measured on gfx950 with one-hot operands). Activation lane group
  // a therefore holds step elements 16 a .. + 15 in bytes 0-15 and
  // 64 + 16 a .. + 15 in bytes 16-31: each weight lane (32 consecutive
  // elements, one block scale) then meets exactly its own 32 activations.
  const uint8_t* arow[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int ar = min(16 * m + r, ti.rows - 1);
    arow[m] = (MODE == 0) ? (const uint8_t*)p.a + (size_t)p.stok[ti.row0 + ar] * K + 16 * g
                          : (const uint8_t*)p.a + (size_t)(ti.row0 + ar) * K + 16 * g;
  }
  const int ncol0 = nt * COLS + wave * COLS_W;
  const uint8_t* brow[FN];   // this lane's 16 code bytes of step 0
  const uint32_t* srow[FN];  // this lane's scale dword of steps 0..3
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const bool up = MODE == 0 && f >= HALF;
    const int n = (MODE == 0) ? ncol0 + (f % HALF) * 16 + r : ncol0 + f * 16 + r;
    const int rb = (n - r) >> 4;
    const uint8_t* W = (const uint8_t*)(up ? p.w1 : p.w0);
    const uint32_t* S = (const uint32_t*)(up ? p.ws1 : p.ws0);
    brow[f] = W + (size_t)ti.e * N * (K / 2) + (size_t)rb * 8 * K + lane * 16;
    srow[f] = S + ((size_t)ti.e * (N / 16) + rb) * (K / 512) * 64 + lane;
  }

  f32x4 acc[MR][FN];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int f = 0; f < FN; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = K / 128;  // a multiple of 4
  Op32 aq[D][MR];
  u32x4 bq[D][FN];
  uint32_t sq[D][FN];
  auto load_step = [&](int d, int s) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      aq[d][m].lo = ld16(arow[m] + (size_t)s * 128);
      aq[d][m].hi = ld16(arow[m] + (size_t)s * 128 + 64);
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      bq[d][f] = ld16_nt(brow[f] + (size_t)s * 1024);
      sq[d][f] = srow[f][(s >> 2) * 64] >> (8 * (s & 3));
    }
  };
  auto consume = [&](int d) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      i32x8 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = (int)aq[d][m].lo[i];
        a[4 + i] = (int)aq[d][m].hi[i];
      }
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        i32x8 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b[i] = (int)bq[d][f][i];
          b[4 + i] = 0;
        }
        acc[m][f] = mfma_fp8_fp4(a, b, (int)(sq[d][f] & 0xffu), acc[m][f]);
      }
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load_step(d, min(d, nks - 1));
  int s0 = 0;
  for (; s0 + 2 * D <= nks; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      consume(d);
      load_step(d, s0 + d + D);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (s0 + d < nks) {
      consume(d);
      if (s0 + d + D < nks) load_step(d, s0 + d + D);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (s0 + D + d < nks) consume(d);

  if (MODE == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * m + 4 * g + i;
        const bool valid = row < ti.rows;
        const float xs = valid ? p.a_scale[p.stok[ti.row0 + row]] : 0.f;
        float rowmax = 0.f;
#pragma unroll
        for (int f = 0; f < HALF; ++f) {
          const int n = ncol0 + f * 16 + r;
          if (valid) {
            const float h = silu_f32(acc[m][f][i] * xs) * (acc[m][f + HALF][i] * xs);
            const float hs = store_h(p, (size_t)(ti.row0 + row) * N + n, h);
            rowmax = fmaxf(rowmax, fabsf(hs));
          }
        }
        row_amax_update(p.hamax, ti.row0 + row, rowmax, valid);
      }
    }
  } else {
    uint16_t* out = (uint16_t*)p.out;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * m + 4 * g + i;
        if (row < ti.rows) {
          const float rs = p.a_scale[ti.row0 + row] * p.sw[ti.row0 + row];
#pragma unroll
          for (int f = 0; f < FN; ++f) {
            const int n = ncol0 + f * 16 + r;
            out[(size_t)(ti.row0 + row) * N + n] = (uint16_t)f32_to_bf16_bits(acc[m][f][i] * rs);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- tiled variant
// An LDS tile row holds 128 bytes of k (64 bf16 or 128 fp8 values) as eight
// 16-byte chunks; chunk c of row r lives at chunk position c ^ (r & 7), so the
// 16 rows of one MFMA operand read spread over all banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int MODE, typename AT, bool FP8, bool PACKED>
__global__ __launch_bounds__(256, 2) void gemm_tiled_kernel(GemmArgs p) {
  using WT = typename WTraits<FP8>::W;
  constexpr int BM = kTiledBM, NBR = 128;
  constexpr int BK = FP8 ? 128 : 64;           // k values per stage (128 bytes per row)
  constexpr int A_BYTES = BM * 128, B_BYTES = NBR * 128, STAGE = A_BYTES + B_BYTES;
  constexpr int COLS = (MODE == 0) ? 64 : 128;  // output columns per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int ntn = p.N / COLS;
  const int mt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  TileInfo ti;
  if (!tile_info(p, mt, BM, ti)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1, r = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N;
  const int n0 = nt * COLS;
  constexpr int CH = BK / 8;  // values per 16-byte LDS chunk of A: bf16 8, fp8 16

  // Global -> LDS assignment: 1024 chunks of A and of B per stage, 4 each per thread.
  const AT* agp[4];
  const WT* bgp[4];
  int soff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, lr = q >> 3, c = q & 7;
    const int ar = min(lr, ti.rows - 1);
    agp[i] = (MODE == 0) ? (const AT*)p.a + (size_t)p.stok[ti.row0 + ar] * K + c * CH
                         : (const AT*)p.a + (size_t)(ti.row0 + ar) * K + c * CH;
    const WT* W;
    int n;
    if (MODE == 0) {
      W = (const WT*)(lr < 64 ? p.w0 : p.w1);
      n = n0 + (lr & 63);
    } else {
      W = (const WT*)p.w0;
      n = n0 + lr;
    }
    soff[i] = swz(lr, c);
    if (PACKED) {
      // The stage's B tile is 8 row blocks x (128 bytes of k) of fragment
      // blocks; chunk q of it is 16 contiguous bytes, and it goes to LDS
      // linearly at q * 16. Row block rb = q / 128 covers tile rows 16 rb..
      const int rb = q >> 7, within = q & 127;
      const int nb = (MODE == 0) ? n0 + 16 * (rb & 3) : n0 + 16 * rb;
      const WT* Wb = (const WT*)((MODE == 0) ? (rb < 4 ? p.w0 : p.w1) : p.w0);
      bgp[i] = Wb + (size_t)ti.e * N * K + (size_t)(nb >> 4) * 16 * K + within * CH;
      boff[i] = q * 16;
    } else {
      bgp[i] = W + ((size_t)ti.e * N + n) * K + c * CH;
      boff[i] = soff[i];
    }
  }

  int arow_l[4], brow_l[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    arow_l[f] = wm * 64 + f * 16 + r;
    brow_l[f] = (MODE == 0) ? ((f < 2) ? wn * 32 + f * 16 + r : 64 + wn * 32 + (f - 2) * 16 + r)
                            : wn * 64 + f * 16 + r;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  using AL = typename std::conditional<FP8, ALoad16<uint16_t>, ALoad16<AT>>::type;
  AL ra[4];
  u32x4 rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (FP8)
        ra[i].v = ld16(agp[i] + (size_t)kt * BK);
      else
        ra[i].load(agp[i] + (size_t)kt * BK);
      rb[i] = ld16(bgp[i] + (size_t)kt * (PACKED ? 16 * BK : BK));
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st16(base + soff[i], ra[i].bits());
      st16(base + A_BYTES + boff[i], rb[i]);
    }
  };

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* As = smem + buf * STAGE;
    const uint8_t* Bs = As + A_BYTES;
    if constexpr (FP8) {
      // one 16x16x128 MFMA per stage: lane group g holds chunks 2g and 2g+1
      Op32 af[4], bfr[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        af[f].lo = ld16(As + swz(arow_l[f], 2 * g));
        af[f].hi = ld16(As + swz(arow_l[f], 2 * g + 1));
        if (PACKED) {  // fragment block of row block brow_l / 16: 64 lanes x 32 bytes
          const uint8_t* blk = Bs + (brow_l[f] >> 4) * 2048 + lane * 32;
          bfr[f].lo = ld16(blk);
          bfr[f].hi = ld16(blk + 16);
        } else {
          bfr[f].lo = ld16(Bs + swz(brow_l[f], 2 * g));
          bfr[f].hi = ld16(Bs + swz(brow_l[f], 2 * g + 1));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_op(af[i], bfr[j], acc[i][j]);
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 af[4], bfr[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          af[f] = ld16(As + swz(arow_l[f], s * 4 + g));
          // packed: row block brow_l / 16 holds two 1 KB k-step blocks per stage
          bfr[f] = PACKED ? ld16(Bs + ((brow_l[f] >> 4) * 2 + s) * 1024 + lane * 16)
                          : ld16(Bs + swz(brow_l[f], s * 4 + g));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma_op(af[i], bfr[j], acc[i][j]);
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  if (MODE == 0) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + fm * 16 + 4 * g + i;
        const bool valid = row < ti.rows;
        float rowmax = 0.f;
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
          const int n = n0 + wn * 32 + fn * 16 + r;
          if (valid) {
            const float h = gateup_value<FP8>(p, ti, row, n, acc[fm][fn][i], acc[fm][fn + 2][i]);
            const float hs = store_h(p, (size_t)(ti.row0 + row) * N + n, h);
            rowmax = fmaxf(rowmax, fabsf(hs));
          }
        }
        if constexpr (FP8) row_amax_update(p.hamax, ti.row0 + row, rowmax, valid);
      }
  } else {
    uint16_t* out = (uint16_t*)p.out;
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + fm * 16 + 4 * g + i;
        if (row < ti.rows) {
#pragma unroll
          for (int fn = 0; fn < 4; ++fn) {
            const int n = n0 + wn * 64 + fn * 16 + r;
            out[(size_t)(ti.row0 + row) * N + n] =
                (uint16_t)f32_to_bf16_bits(down_value<FP8>(p, ti, row, n, acc[fm][fn][i]));
          }
        }
      }
  }
}

// Epilogue of the transposed tiles (wide and DMA variants). acc[fm][fn]
// holds, in lane (r, g), output row row_base + 16 fm + r and the 4 output
// columns 16 c(fn) + 4 g .. + 3, where c(fn) is the fragment's column block:
// gate/up: fn < FN / 2 gate and fn + FN / 2 the matching up block,
// c = (FN / 2) wn + fn; down: c = FN wn + fn.
template <int MODE, bool FP8, int FM, int FN, bool BLOCK_SCALED = false>
__device__ __forceinline__ void transposed_epilogue(const GemmArgs& p, const TileInfo& ti,
                                                    const f32x4 (&acc)[FM][FN], int row_base,
                                                    int n0, int wn, int r, int g) {
  const int N = p.N;
  constexpr int NF = (MODE == 0) ? FN / 2 : FN;  // output column blocks of this wave
  // fp8: per-column weight scales of this lane's 4 columns, loaded once
  f32x4 cs0[NF], cs1[NF];
#pragma unroll
  for (int fn = 0; fn < NF; ++fn) {
    cs0[fn] = cs1[fn] = f32x4{1.f, 1.f, 1.f, 1.f};
    if constexpr (FP8 && !BLOCK_SCALED) {  // MXFP4: the block scales act inside the MFMA
      const int n = n0 + (wn * NF + fn) * 16 + 4 * g;
      const size_t c = (size_t)ti.e * N + n;
      cs0[fn] = __builtin_bit_cast(f32x4, ld16(p.ws0 + c));
      if constexpr (MODE == 0) cs1[fn] = __builtin_bit_cast(f32x4, ld16(p.ws1 + c));
    }
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int row = row_base + fm * 16 + r;
    const bool valid = row < ti.rows;
    const size_t orow = (size_t)(ti.row0 + (valid ? row : 0)) * N;
    if constexpr (MODE == 0) {
      // fp8: the token's activation scale
      const float xs = (FP8 && valid) ? p.a_scale[p.stok[ti.row0 + row]] : 1.f;
      float rowmax = 0.f;
#pragma unroll
      for (int fn = 0; fn < NF; ++fn) {
        const int n = n0 + (wn * NF + fn) * 16 + 4 * g;
        float h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float gv = acc[fm][fn][i], uv = acc[fm][fn + NF][i];
          if constexpr (FP8) {
            gv = gv * xs * cs0[fn][i];
            uv = uv * xs * cs1[fn][i];
          }
          h[i] = valid ? silu_f32(gv) * uv : 0.f;
        }
        // h is stored as bf16 (round to nearest even); the quantised paths
        // take the row's max |h| over the stored values
        const u32x2 hb = u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        if constexpr (FP8) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
            rowmax = fmaxf(rowmax, fmaxf(fabsf(bf16_bits_to_f32(hb[i] & 0xffffu)),
                                         fabsf(bf16_bits_to_f32(hb[i] >> 16))));
        }
        if (valid) *reinterpret_cast<u32x2*>((uint16_t*)p.out + orow + n) = hb;
      }
      if constexpr (FP8) {
        // the row's 32 columns of this wave sit in lanes r, r + 16, r + 32, r + 48
        rowmax = fmaxf(rowmax, __shfl_xor(rowmax, 16));
        rowmax = fmaxf(rowmax, __shfl_xor(rowmax, 32));
        if (valid && g == 0) atomicMax(&p.hamax[ti.row0 + row], __float_as_uint(rowmax));
      }
    } else {
      if (valid) {
        // rsf * routing weight of the row (fp8: times the row's activation scale)
        float rs = p.sw ? p.sw[ti.row0 + row] : 1.f;  // no per-row scale: input gradients
        if constexpr (FP8) rs = p.a_scale[ti.row0 + row] * rs;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int n = n0 + (wn * FN + fn) * 16 + 4 * g;
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = FP8 ? acc[fm][fn][i] * cs0[fn][i] * rs : acc[fm][fn][i] * rs;
          *reinterpret_cast<u32x2*>((uint16_t*)p.out + orow + n) =
              u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
      }
    }
  }
}

// M-tiles per ordering group of the wide and DMA variants: the 32 blocks that
// run together on one XCD cover 4 M-tiles x 8 N-tiles of an expert, so each
// A slice is shared by 8 of them and each weight slice by 4 in the XCD's L2.
constexpr int kGroupM = 4;

// Tiles per XCD chunk in xcd_chunked_tile.
constexpr int kXcdChunk = 32;

// Tile taken by workgroup b of a grouped GEMM over n_tiles numbered tiles.
// Workgroups go to the 8 XCDs round-robin (b % 8). Chunks of kXcdChunk
// consecutive tiles are dealt to the XCDs in turn: the blocks running
// together on one XCD (32 CUs) take one chunk and share its operands in that
// XCD's L2, and the 8 XCDs together work on 256 consecutive tiles. So one
// expert's tiles run on the whole chip at once, and its weights and rows
// (about 160 MB for an expert of 10K rows) stay in the 256 MB MALL between
// its M-tile groups; a contiguous share per XCD would run eight experts at
// once, whose re-reads would miss the MALL. Tiles of the last, partial round
// of 256 go round-robin.
__device__ __forceinline__ int xcd_chunked_tile(int b, int n_tiles) {
  constexpr int R = 8 * kXcdChunk;
  if (b >= n_tiles / R * R) return b;
  const int q = b >> 3;  // the block's place on its XCD
  return ((q / kXcdChunk) * 8 + (b & 7)) * kXcdChunk + q % kXcdChunk;
}

// ---------------------------------------------------------------- wide variant
// Prefill with packed weights. A workgroup of 8 waves (two per SIMD) computes
// BM rows x 256 weight rows (gate/up: 128 gate + 128 up columns; down: 256
// columns) over K in stages of 128 bytes of k, double buffered in LDS (A
// swizzled row-major, B as the packed fragment blocks read back in lane
// order). Waves form a 2 x 4 grid: BM = 256 -> 128 x 64 per wave (32
// fragments), BM = 128 -> 64 x 64 (16 fragments). Every k-step loads all of a
// wave's operand fragments before its MFMAs; the second wave on the SIMD
// covers the LDS latency.
//
// Tile order: the active (M-tile, N-tile) pairs are numbered expert by
// expert, in blocks of kGroupM M-tiles, N-tile-major inside a block, and
// dealt to the XCDs in chunks (xcd_chunked_tile), so blocks running together
// on one XCD share A and weight slices in that XCD's L2.
//
// The MFMAs compute the transposed tile (weight fragment as the A operand):
// each lane then holds 4 consecutive output columns of one row, stored as
// one 8-byte (bf16) or 16-byte (fp32) write.
template <int MODE, typename AT, bool FP8, int BM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_wide_kernel(GemmArgs p) {
  using WT = typename WTraits<FP8>::W;
  constexpr int BK = FP8 ? 128 : 64;          // k values per stage (128 bytes per row)
  constexpr int CH = BK / 8;                  // values per 16-byte chunk
  constexpr int A_BYTES = BM * 128, B_BYTES = 256 * 128, STAGE = A_BYTES + B_BYTES;
  constexpr int FM = BM / 32, FN = 4;         // fragments per wave along M / N
  constexpr int COLS = (MODE == 0) ? 128 : 256;
  constexpr int AQ = BM / 64;                 // A chunks per thread per stage
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int ntn = p.N / COLS;
  const int n_tiles = p.meta[0] * ntn;
  const int b = blockIdx.x;
  if (b >= n_tiles) return;
  const int j = xcd_chunked_tile(b, n_tiles);
  const int e = p.tile_e[j / ntn];
  const int ts = p.e_tstart[e], nm = p.e_ntiles[e];
  const int jj = j - ts * ntn;
  // inside the expert: blocks of kGroupM M-tiles, N-tile-major inside a block
  const int mb = jj / (kGroupM * ntn), rem = jj - mb * kGroupM * ntn;
  const int gm = min(kGroupM, nm - mb * kGroupM);
  const int nt = rem / gm, mt = ts + mb * kGroupM + rem % gm;
  TileInfo ti;
  ti.e = e;
  ti.row0 = p.tile_r[mt];
  ti.rows = min(BM, p.offsets[e + 1] - ti.row0);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3, r = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N;
  const int n0 = nt * COLS;

  // A: AQ chunks per thread; chunk q = tid + 512 i -> tile row q / 8, chunk q % 8.
  const AT* agp[AQ];
  int aoff[AQ];
#pragma unroll
  for (int i = 0; i < AQ; ++i) {
    const int q = tid + 512 * i, lr = q >> 3, c = q & 7;
    const int ar = min(lr, ti.rows - 1);
    agp[i] = (MODE == 0) ? (const AT*)p.a + (size_t)p.stok[ti.row0 + ar] * K + c * CH
                         : (const AT*)p.a + (size_t)(ti.row0 + ar) * K + c * CH;
    aoff[i] = swz(lr, c);
  }
  // B: 4 chunks per thread; chunk q = tid + 512 i -> row block q / 128 of the
  // tile (16 blocks; MODE 0: gate 0..7 then up 8..15), 16 bytes (q % 128) of
  // its stage block. Row block of chunk i: (tid >> 7) + 4 i.
  const WT* bgp[4];
  {
    const size_t eoff = (size_t)ti.e * N * K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rbk = (tid >> 7) + 4 * i;
      const WT* W = (const WT*)((MODE == 0 && rbk >= 8) ? p.w1 : p.w0);
      const int blk = (MODE == 0) ? (n0 >> 4) + (rbk & 7) : (n0 >> 4) + rbk;
      bgp[i] = W + eoff + (size_t)blk * 16 * K + (tid & 127) * CH;
    }
  }

  int arow_l[FM], brbl[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) arow_l[f] = wm * (BM / 2) + f * 16 + r;
#pragma unroll
  for (int f = 0; f < FN; ++f)
    brbl[f] = (MODE == 0) ? ((f < 2) ? wn * 2 + f : 8 + wn * 2 + (f - 2)) : wn * 4 + f;
  // Waves whose rows are all padding skip their MFMAs (uniform per wave).
  const bool live = wm * (BM / 2) < ti.rows;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  using AL = typename std::conditional<FP8, ALoad16<uint16_t>, ALoad16<AT>>::type;
  AL ra[AQ];
  u32x4 rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < AQ; ++i) {
      if constexpr (FP8)
        ra[i].v = ld16(agp[i] + (size_t)kt * BK);
      else
        ra[i].load(agp[i] + (size_t)kt * BK);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = ld16(bgp[i] + (size_t)kt * 16 * BK);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < AQ; ++i) st16(base + aoff[i], ra[i].bits());
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(base + A_BYTES + ((tid >> 7) + 4 * i) * 2048 + (tid & 127) * 16, rb[i]);
  };

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* As = smem + buf * STAGE;
    const uint8_t* Bs = As + A_BYTES;
    if (live) {
      if constexpr (FP8) {
        Op32 af[FM], bfr[FN];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const uint8_t* blk = Bs + brbl[f] * 2048 + lane * 32;
          bfr[f].lo = ld16(blk);
          bfr[f].hi = ld16(blk + 16);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          af[i].lo = ld16(As + swz(arow_l[i], 2 * g));
          af[i].hi = ld16(As + swz(arow_l[i], 2 * g + 1));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jn = 0; jn < FN; ++jn) acc[i][jn] = mfma_op(bfr[jn], af[i], acc[i][jn]);
      } else {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          u32x4 af[FM], bfr[FN];
#pragma unroll
          for (int f = 0; f < FN; ++f) bfr[f] = ld16(Bs + (brbl[f] * 2 + s) * 1024 + lane * 16);
#pragma unroll
          for (int i = 0; i < FM; ++i) af[i] = ld16(As + swz(arow_l[i], s * 4 + g));
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jn = 0; jn < FN; ++jn) acc[i][jn] = mfma_op(bfr[jn], af[i], acc[i][jn]);
        }
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  transposed_epilogue<MODE, FP8, FM, FN>(p, ti, acc, wm * (BM / 2), n0, wn, r, g);
}

// ---------------------------------------------------------------- DMA variant
// Prefill with packed bf16 weights and bf16 A. Same tile shape, wave grid and
// tile order as the wide variant, but operands go from global memory straight
// into LDS (global_load_lds, 16 bytes per lane, no staging registers) through
// a ring of NS stages of one 32-k matrix-core step each, filled NS-1 stages
// ahead, so roughly three stages of loads are in flight while one is
// computed. Waits are explicit: before stage kt is read, vmcnt leaves only
// the DMAs of the later stages outstanding, and a raw barrier publishes every
// wave's stage-kt DMAs. Each wave has every LDS read of a stage completed
// before the barrier that lets that stage buffer be refilled. Fragment reads
// run a batch ahead of the MFMAs (see the k loop), so the matrix core keeps
// working while the next fragments arrive. A wave
// whose rows are partly past the expert's last row runs a copy of the loop
// that reads and multiplies only its first FM/4 or FM/2 fragments (none if
// no row is live), so an expert slightly over a tile boundary costs little
// matrix-core time in a 256-row tile.
//
// LDS per stage: A is BM rows x 64 bytes, row r's chunk g (16 bytes) stored at
// position g ^ ((r >> 1) & 3) so the 16 rows of a fragment read hit distinct
// banks; B is 16 row blocks x 1 KB in the packed fragment order.

//
// Modes: 0 gate/up (A = x rows through the sorted token list, B = the gate and
// up matrices side by side, out = h); 1 down (A = h rows, out = rsf * w * y).
// The backward pass adds: 2 gate/up again, storing the pre-activations g | u
// in fp32 (and h transposed for the weight gradients); 3 the gradient through the
// down projection and SwiGLU (A = dout rows through the sorted token list,
// B = W_down transposed, out = dg | du); 4 the input gradient of every row
// (A = dg | du rows, B = W_gate transposed for the first half of k and W_up
// transposed for the second, out = dx rows).
constexpr bool mode_paired(int m) { return m == 0 || m == 2; }
constexpr bool mode_gathered(int m) { return m == 0 || m == 2 || m == 3; }

template <int MODE, int FM, int FN>
__device__ __forceinline__ void backward_epilogue(const GemmArgs& p, const TileInfo& ti,
                                                  const f32x4 (&acc)[FM][FN], int row_base,
                                                  int n0, int nt, int wn, int r, int g);

template <int MODE, int BM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_dma_kernel(GemmArgs p) {
  constexpr int NS = 4;                        // stages in the ring
  constexpr int A_BYTES = BM * 64, B_BYTES = 256 * 64, STAGE = A_BYTES + B_BYTES;
  constexpr int FM = BM / 32, FN = 4;
  constexpr bool PAIRED = mode_paired(MODE);
  constexpr int COLS = PAIRED ? 128 : 256;
  constexpr int AI = BM / 128;                 // A DMA instructions per wave per stage
  static_assert(AI == 1 || AI == 2, "row groups per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

  const int ntn = p.N / COLS;
  const int n_tiles = p.meta[0] * ntn;
  const int b = blockIdx.x;
  if (b >= n_tiles) return;
  const int j = xcd_chunked_tile(b, n_tiles);
  const int e = p.tile_e[j / ntn];
  const int ts = p.e_tstart[e], nm = p.e_ntiles[e];
  const int jj = j - ts * ntn;
  // inside the expert: blocks of kGroupM M-tiles, N-tile-major inside a block
  const int mb = jj / (kGroupM * ntn), rem = jj - mb * kGroupM * ntn;
  const int gm = min(kGroupM, nm - mb * kGroupM);
  const int nt = rem / gm, mt = ts + mb * kGroupM + rem % gm;
  TileInfo ti;
  ti.e = e;
  ti.row0 = p.tile_r[mt];
  ti.rows = min(BM, p.offsets[e + 1] - ti.row0);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3, r = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N;
  const int n0 = nt * COLS;

  // A DMA sources: instruction i of this wave fills tile rows 16 * (wave * AI + i) ..;
  // lane l writes LDS row l / 4, position l % 4, which holds chunk (l % 4) ^ ((row >> 1) & 3).
  const uint16_t* asrc[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (wave * AI + i) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 1) & 3);
    const int ar = min(row, ti.rows - 1);
    const uint16_t* base = mode_gathered(MODE)
                               ? (const uint16_t*)p.a + (size_t)p.stok[ti.row0 + ar] * K
                               : (const uint16_t*)p.a + (size_t)(ti.row0 + ar) * K;
    asrc[i] = base + chunk * 8;
  }
  // B DMA sources: instruction i fills row block wave * 2 + i (paired modes:
  // 0..7 gate, 8..15 up). Mode 4 reads w0 for the first half of k and w1 for
  // the second, each a [N, K / 2] matrix.
  constexpr bool KSPLIT = MODE == 4;
  const int KB = KSPLIT ? K / 2 : K;  // reduction length of one weight matrix
  const uint16_t* bsrc[2];
  const uint16_t* bsrc2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rbk = wave * 2 + i;
    const uint16_t* W = (const uint16_t*)((PAIRED && rbk >= 8) ? p.w1 : p.w0);
    const int blk = PAIRED ? (n0 >> 4) + (rbk & 7) : (n0 >> 4) + rbk;
    const size_t off = (size_t)ti.e * N * KB + (size_t)blk * 16 * KB + lane * 8;
    bsrc[i] = W + off;
    bsrc2[i] = KSPLIT ? (const uint16_t*)p.w1 + off : nullptr;
  }
  const int kh = KB / 32;  // k-steps per weight matrix
  // DMA of k-step kt into ring slot kt % NS: this wave's first AL row groups
  // of A (the others lie past the expert's last row and are not loaded) and
  // its two weight row blocks.
  auto issue = [&](int kt, auto al_c) {
    constexpr int AL = decltype(al_c)::value;
    uint8_t* st = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < AL; ++i)
      dma16(asrc[i] + (size_t)kt * 32, st + (wave * AI + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint16_t* bp = (!KSPLIT || kt < kh) ? bsrc[i] + (size_t)kt * 512
                                                : bsrc2[i] + (size_t)(kt - kh) * 512;
      dma16(bp, st + A_BYTES + (wave * 2 + i) * 1024);
    }
  };

  int aoff[FM], boff[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int row = wm * (BM / 2) + f * 16 + r;
    aoff[f] = row * 64 + ((g ^ ((row >> 1) & 3)) << 4);
  }
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int rbl = PAIRED ? ((f < 2) ? wn * 2 + f : 8 + wn * 2 + (f - 2)) : wn * 4 + f;
    boff[f] = A_BYTES + rbl * 1024 + lane * 16;
  }
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / 32;  // >= 4 since K is a multiple of 128
  // The k loop for a wave whose live rows fit in its first NF fragments
  // (NF = 0: a wave with no live rows only takes part in the loads and
  // barriers) and that loads AL of its AI row groups of A. Every variant
  // passes the same barriers; each waits for its own loads only.
  auto kloop = [&](auto nf_c, auto al_c) {
    constexpr int NF = decltype(nf_c)::value;
    constexpr int PER = decltype(al_c)::value + 2;  // this wave's DMAs per stage
#pragma unroll
    for (int s0 = 0; s0 < NS - 1; ++s0) issue(s0, al_c);
    if constexpr (NF > 0) {
      // Fragment reads run one batch ahead of the multiplies: the A fragments
      // of batch b + 1 are read while the MFMAs of batch b execute, and the B
      // fragments and first A batch of step kt + 1 while the last batch of
      // step kt executes (B double-buffered). Each wait for a batch's reads
      // then comes after they have had a batch of MFMAs to land.
      constexpr int AB = NF >= 2 ? 2 : 1;  // A fragments per batch
      constexpr int NB = NF / AB;
      u32x4 af[NF], bq0[FN], bq1[FN];
      auto wait_stage = [&](int s) {  // stage s landed for this wave
        if (s + NS - 2 < nk)
          wait_vmcnt<(NS - 2) * PER>();
        else
          wait_vmcnt<0>();
      };
      auto batch = [&](int b0, const u32x4(&bq)[FN]) {
#pragma unroll
        for (int i = b0; i < b0 + AB; ++i)
#pragma unroll
          for (int jn = 0; jn < FN; ++jn) acc[i][jn] = mfma_op(bq[jn], af[i], acc[i][jn]);
      };
      auto step = [&](int kt, const u32x4(&bc)[FN], u32x4(&bn)[FN], auto more_c) {
        constexpr bool MORE = decltype(more_c)::value;
        const uint8_t* st = smem + (kt % NS) * STAGE;
#pragma unroll
        for (int b = 0; b < NB - 1; ++b) {
          batch(b * AB, bc);
#pragma unroll
          for (int i = (b + 1) * AB; i < (b + 2) * AB; ++i) af[i] = ld16(st + aoff[i]);
          // one read after each of the first AB MFMAs, the rest of the batch after
#pragma unroll
          for (int i = 0; i < AB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, AB * FN - AB, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (MORE) {
          // every read of slot kt is done (its last batch is in registers), so
          // after the barrier the slot can be refilled and step kt + 1 read
          asm volatile("" ::: "memory");
          wait_lgkmcnt0();
          wait_stage(kt + 1);
          barrier_only();
          asm volatile("" ::: "memory");
          if (kt + NS < nk) issue(kt + NS, al_c);
          __builtin_amdgcn_sched_barrier(0);
          const uint8_t* sn = smem + ((kt + 1) % NS) * STAGE;
          batch((NB - 1) * AB, bc);
#pragma unroll
          for (int f = 0; f < FN; ++f) bn[f] = ld16(sn + boff[f]);
#pragma unroll
          for (int i = 0; i < AB; ++i) af[i] = ld16(sn + aoff[i]);
#pragma unroll
          for (int i = 0; i < FN + AB; ++i) {
            if (i < AB * FN) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if (FN + AB < AB * FN)
            __builtin_amdgcn_sched_group_barrier(0x008, AB * FN - FN - AB, 0);
          __builtin_amdgcn_sched_barrier(0);
        } else {
          batch((NB - 1) * AB, bc);
        }
      };
      wait_stage(0);
      barrier_only();
      asm volatile("" ::: "memory");
      if (NS - 1 < nk) issue(NS - 1, al_c);
#pragma unroll
      for (int f = 0; f < FN; ++f) bq0[f] = ld16(smem + boff[f]);
#pragma unroll
      for (int i = 0; i < AB; ++i) af[i] = ld16(smem + aoff[i]);
      // nk is a multiple of 4: steps in pairs, B buffers alternating
      for (int kt = 0; kt < nk - 2; kt += 2) {
        step(kt, bq0, bq1, std::true_type{});
        step(kt + 1, bq1, bq0, std::true_type{});
      }
      step(nk - 2, bq0, bq1, std::true_type{});
      step(nk - 1, bq1, bq0, std::false_type{});
    } else {
      // no live rows: the wave only loads and passes the same barriers
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + NS - 2 < nk)
          wait_vmcnt<(NS - 2) * PER>();
        else
          wait_vmcnt<0>();
        barrier_only();
        asm volatile("" ::: "memory");
        if (kt + NS - 1 < nk) issue(kt + NS - 1, al_c);
      }
    }
  };
  // fragments of this wave that hold live rows, and its A row groups with
  // live rows (row groups 16 (wave AI + i) ..)
  const int need = min(FM, max(0, (ti.rows - wm * (BM / 2) + 15) >> 4));
  const int al = min(AI, max(0, (ti.rows - wave * AI * 16 + 15) >> 4));
  auto run = [&](auto nf_c) {
    if (al == 0)
      kloop(nf_c, std::integral_constant<int, 0>{});
    else if (al == 1)
      kloop(nf_c, std::integral_constant<int, 1>{});
    else
      kloop(nf_c, std::integral_constant<int, AI>{});
  };
  if (need == 0)
    run(std::integral_constant<int, 0>{});
  else if (need <= FM / 4)
    run(std::integral_constant<int, FM / 4>{});
  else if (need <= FM / 2)
    run(std::integral_constant<int, FM / 2>{});
  else
    run(std::integral_constant<int, FM>{});

  if constexpr (MODE <= 1)
    transposed_epilogue<MODE, false, FM, FN>(p, ti, acc, wm * (BM / 2), n0, wn, r, g);
  else if constexpr (MODE == 4)
    transposed_epilogue<1, false, FM, FN>(p, ti, acc, wm * (BM / 2), n0, wn, r, g);
  else
    backward_epilogue<MODE, FM, FN>(p, ti, acc, wm * (BM / 2), n0, nt, wn, r, g);
}

// Epilogues of modes 2 and 3 (lane (r, g) of fragment (fm, fn) holds row
// row_base + 16 fm + r, columns 16 c + 4 g .. + 3 as in transposed_epilogue).
// Transposed copies (h, dg, du) are [N, pcols] matrices whose column of
// sorted row q is p.pcol[e] + q - offsets[e] (each expert's rows a segment),
// stored in 32-column blocks: element (n, c) at ((c / 32) N + n) 32 + c % 32.
__device__ __forceinline__ void store_col4(uint16_t* base, int N, int n, int col,
                                           const float (&v)[4]) {
  uint16_t* p = base + ((((size_t)(col >> 5) * N) + n) << 5) + (col & 31);
#pragma unroll
  for (int i = 0; i < 4; ++i) p[32 * i] = (uint16_t)f32_to_bf16_bits(v[i]);
}

template <int MODE, int FM, int FN>
__device__ __forceinline__ void backward_epilogue(const GemmArgs& p, const TileInfo& ti,
                                                  const f32x4 (&acc)[FM][FN], int row_base,
                                                  int n0, int nt, int wn, int r, int g) {
  const int N = p.N;
  const size_t ld = 2 * (size_t)N;  // row length of the g | u (fp32) and dg | du (bf16) matrices
  uint16_t* out = (uint16_t*)p.out;
  const bool tr = p.tout0 != nullptr;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int row = row_base + fm * 16 + r;
    const bool valid = row < ti.rows;
    const size_t grow = (size_t)(ti.row0 + (valid ? row : 0));
    const int col = tr ? p.pcol[ti.e] + (int)grow - p.offsets[ti.e] : 0;
    if constexpr (MODE == 2) {
      constexpr int NF = FN / 2;
      if (valid) {
#pragma unroll
        for (int fn = 0; fn < NF; ++fn) {
          const int n = n0 + (wn * NF + fn) * 16 + 4 * g;
          const f32x4 gv = acc[fm][fn], uv = acc[fm][fn + NF];
          float* gu = (float*)p.out + grow * ld;
          st16(gu + n, __builtin_bit_cast(u32x4, gv));
          st16(gu + N + n, __builtin_bit_cast(u32x4, uv));
          if (tr) {
            float h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = silu_f32(gv[i]) * uv[i];
            store_col4((uint16_t*)p.tout0, N, n, col, h);
          }
        }
      }
    } else {
      // dh = rsf * w * q; du = dh * silu(g); dg = dh * u * silu'(g); the row's
      // share of sum_n h q for the routing-weight gradient
      const float sw = valid ? p.sw[grow] : 0.f;
      const float* gu = (const float*)p.a2 + grow * ld;
      float hq = 0.f;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + (wn * FN + fn) * 16 + 4 * g;
        if (valid) {
          const f32x4 gg = __builtin_bit_cast(f32x4, ld16(gu + n));
          const f32x4 uu = __builtin_bit_cast(f32x4, ld16(gu + N + n));
          float dg[4], du[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float q = acc[fm][fn][i];
            const float sg = sigmoid_f32(gg[i]);
            const float a = gg[i] * sg;
            const float dh = sw * q;
            du[i] = dh * a;
            dg[i] = dh * uu[i] * (sg * (1.f + gg[i] * (1.f - sg)));
            hq += a * uu[i] * q;
          }
          *reinterpret_cast<u32x2*>(out + grow * ld + n) =
              u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
          *reinterpret_cast<u32x2*>(out + grow * ld + N + n) =
              u32x2{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
          if (tr) {
            store_col4((uint16_t*)p.tout0, N, n, col, dg);
            store_col4((uint16_t*)p.tout1, N, n, col, du);
          }
        }
      }
      // the 4 lanes of a row (g = 0..3) hold its other columns of this wave
      hq += __shfl_xor(hq, 16);
      hq += __shfl_xor(hq, 32);
      if (valid && g == 0) p.part[grow * p.nparts + nt * 4 + wn] = hq;
    }
  }
}

// ---------------------------------------------------------------- fp8 DMA variant
// Prefill with packed E4M3 weights and E4M3 A (x or h codes, per-row scales
// applied in the epilogue). One matrix-core step is 128 k (16x16x128 fp8),
// loaded as two half-stages of 64 k: A is TM rows x 64 bytes (chunk g of row
// r at position g ^ ((r >> 1) & 3)), B is the first or second KB of each of
// the tile's 16-row weight blocks' 2 KB fragment blocks (lanes 0-31 of a
// fragment hold k 0..63, lanes 32-63 k 64..127). The ring has NS half-stage
// slots and is filled NS - 2 half-stages ahead, so the two halves being read
// are never refilled: the slot refilled at half-stage i last held half-stage
// i - 2, read by the step that ended before barrier i. Lanes 0-31 read their
// operands from the step's first half, lanes 32-63 from its second.
//
// Tile shapes (8 waves, each 16 FM rows x 4 weight blocks, FM = 8 or 4):
//   TM = 128 or 256: 2 x 4 waves over 16 weight blocks (gate/up: 128 output
//     columns, 8 gate + 8 up blocks; down: 256 columns);
//   TM = 512: 4 x 2 waves over 8 weight blocks (gate/up: 64 columns; down:
//     128), for experts with more than 256 rows: the tile holds all of such
//     an expert's rows up to 512, so its weights stream from HBM once instead
//     of once per 256-row tile.
template <int MODE, int TM>
struct Dma8Shape {
  static constexpr int WM = TM >= 512 ? 4 : 2;   // waves along the rows
  static constexpr int WN = 8 / WM;              // waves along the weight blocks
  static constexpr int RB = 4 * WN;              // 16-row weight blocks of the tile
  static constexpr int RW = TM / WM;             // rows of one wave
  static constexpr int FM = RW / 16, FN = 4;
  static constexpr int COLS = (MODE == 0) ? RB * 8 : RB * 16;  // output columns
  static constexpr int A_BYTES = TM * 64, B_BYTES = RB * 1024, STAGE = A_BYTES + B_BYTES;
  static constexpr int NS = (160 * 1024) / STAGE;  // 6 (TM 128), 5 (256) or 4 (512) slots
  static constexpr int AHEAD = NS - 2;
  static constexpr int AI = TM / 128;              // A DMA instructions per wave per half-stage
  static constexpr int BI = RB / 8;                // B DMA instructions per wave per half-stage
  static_assert(AHEAD >= 2, "ring too small");
  static_assert(NS * STAGE <= 160 * 1024, "LDS");
};

constexpr int kDma8Lds = 160 * 1024;

// One (M-tile, N-tile) of the fp8 DMA GEMM: rows ti.row0 .. + ti.rows of
// expert ti.e (at most TM), output columns nt * COLS ...
template <int MODE, int TM>
__device__ __forceinline__ void dma8_tile(const GemmArgs& p, const TileInfo& ti, int nt,
                                          uint8_t* smem) {
  using S = Dma8Shape<MODE, TM>;
  constexpr int NS = S::NS, AHEAD = S::AHEAD, STAGE = S::STAGE, A_BYTES = S::A_BYTES;
  constexpr int FM = S::FM, FN = S::FN, AI = S::AI, BI = S::BI, RB = S::RB, RW = S::RW;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / S::WN, wn = wave % S::WN, r = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N;
  const int n0 = nt * S::COLS;

  // A: instruction i of this wave fills tile rows 16 * (wave * AI + i) ..;
  // lane l writes row l / 4, position l % 4 (chunk (l % 4) ^ ((row >> 1) & 3)).
  const uint8_t* asrc[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (wave * AI + i) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 1) & 3);
    const int ar = min(row, ti.rows - 1);
    const uint8_t* base = (MODE == 0) ? (const uint8_t*)p.a + (size_t)p.stok[ti.row0 + ar] * K
                                      : (const uint8_t*)p.a + (size_t)(ti.row0 + ar) * K;
    asrc[i] = base + chunk * 16;
  }
  // B: instruction i fills weight block wave * BI + i (MODE 0: the first RB / 2
  // blocks gate, the others up).
  const uint8_t* bsrc[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int rbk = wave * BI + i;
    const uint8_t* W = (const uint8_t*)((MODE == 0 && rbk >= RB / 2) ? p.w1 : p.w0);
    const int blk = (MODE == 0) ? (n0 >> 4) + rbk % (RB / 2) : (n0 >> 4) + rbk;
    bsrc[i] = W + (size_t)ti.e * N * K + (size_t)blk * 16 * K + lane * 16;
  }
  // half-stage hs (k bytes [64 hs, 64 hs + 64)): this wave's first AL row
  // groups of A (the rest lie past the expert's last row) and its weight blocks
  auto issue = [&](int hs, auto al_c) {
    constexpr int AL = decltype(al_c)::value;
    uint8_t* st = smem + (hs % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < AL; ++i) dma16(asrc[i] + (size_t)hs * 64, st + (wave * AI + i) * 1024);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      dma16_nt(bsrc[i] + (size_t)(hs >> 1) * 2048 + (hs & 1) * 1024,
               st + A_BYTES + (wave * BI + i) * 1024);
  };

  // Operand offsets inside a slot; this lane's half of the step is lane / 32.
  const int half = lane >> 5, c0 = 2 * (g & 1);
  int aoff[FM], boff[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int row = wm * RW + f * 16 + r;
    aoff[f] = row * 64 + ((c0 ^ ((row >> 1) & 3)) << 4);
  }
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int rbl = (MODE == 0) ? ((f < 2) ? wn * 2 + f : RB / 2 + wn * 2 + (f - 2)) : wn * 4 + f;
    boff[f] = A_BYTES + rbl * 1024 + (lane & 31) * 32;
  }
  // the second chunk of a row's 32 bytes sits at position (c0 + 1) ^ swizzle,
  // which is the first position with its lowest bit flipped
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nh = K / 64;  // even, >= 2
  auto kloop = [&](auto nf_c, auto al_c) {
    constexpr int NF = decltype(nf_c)::value;
    constexpr int PER = decltype(al_c)::value + BI;  // this wave's DMAs per half-stage
#pragma unroll
    for (int s0 = 0; s0 < AHEAD; ++s0)
      if (s0 < nh) issue(s0, al_c);
    for (int hs = 0; hs < nh; ++hs) {
      // half-stage hs done for this wave: only later half-stages outstanding
      if (hs + AHEAD - 1 < nh)
        wait_vmcnt<(AHEAD - 1) * PER>();
      else
        wait_vmcnt<0>();
      barrier_only();
      asm volatile("" ::: "memory");
      if (hs + AHEAD < nh) issue(hs + AHEAD, al_c);
      if constexpr (NF > 0) {
        if (hs & 1) {
          const uint8_t* st = smem + ((hs - 1 + half) % NS) * STAGE;
          Op32 af[NF], bfr[FN];
          auto read_a = [&](int i) {
            af[i].lo = ld16(st + aoff[i]);
            af[i].hi = ld16(st + (aoff[i] ^ 16));
          };
#pragma unroll
          for (int f = 0; f < FN; ++f) {
            bfr[f].lo = ld16(st + boff[f]);
            bfr[f].hi = ld16(st + boff[f] + 16);
          }
          read_a(0);
          // A fragment i + 1 is read while the MFMAs of fragment i execute
#pragma unroll
          for (int i = 0; i < NF; ++i) {
#pragma unroll
            for (int jn = 0; jn < FN; ++jn) acc[i][jn] = mfma_op(bfr[jn], af[i], acc[i][jn]);
            if (i + 1 < NF) {
              read_a(i + 1);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, FN - 2, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      wait_lgkmcnt0();
      asm volatile("" ::: "memory");
    }
  };
  const int need = min(FM, max(0, (ti.rows - wm * RW + 15) >> 4));
  const int al = min(AI, max(0, (ti.rows - wave * AI * 16 + 15) >> 4));
  auto run = [&](auto nf_c) {
    if (al == 0)
      kloop(nf_c, std::integral_constant<int, 0>{});
    else if (al == 1)
      kloop(nf_c, std::integral_constant<int, 1>{});
    else
      kloop(nf_c, std::integral_constant<int, AI>{});
  };
  if (need == 0)
    run(std::integral_constant<int, 0>{});
  else if (need <= FM / 4)
    run(std::integral_constant<int, FM / 4>{});
  else if (need <= FM / 2)
    run(std::integral_constant<int, FM / 2>{});
  else
    run(std::integral_constant<int, FM>{});

  transposed_epilogue<MODE, true, FM, FN>(p, ti, acc, wm * RW, n0, wn, r, g);
}

// Every expert in tiles of BM rows (the tile list was built with BM).
template <int MODE, int BM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_dma8_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDma8Lds];
  const int ntn = p.N / Dma8Shape<MODE, BM>::COLS;
  const int n_tiles = p.meta[0] * ntn;
  const int b = blockIdx.x;
  if (b >= n_tiles) return;
  const int j = xcd_chunked_tile(b, n_tiles);
  const int e = p.tile_e[j / ntn];
  const int ts = p.e_tstart[e], nm = p.e_ntiles[e];
  const int jj = j - ts * ntn;
  const int mb = jj / (kGroupM * ntn), rem = jj - mb * kGroupM * ntn;
  const int gm = min(kGroupM, nm - mb * kGroupM);
  const int nt = rem / gm, mt = ts + mb * kGroupM + rem % gm;
  TileInfo ti;
  ti.e = e;
  ti.row0 = p.tile_r[mt];
  ti.rows = min(BM, p.offsets[e + 1] - ti.row0);
  dma8_tile<MODE, BM>(p, ti, nt, smem);
}

// Mixed tile heights (the tile list was built with kMixedBM): an expert with
// up to 256 rows runs 256-row tiles of COLS(256) columns; an expert with more
// runs 512-row tiles (two list slots each) of COLS(256) / 2 columns, twice as
// many of them, so every expert has (slots x N / COLS(256)) units and unit j
// belongs to slot j / (N / COLS(256)) as with uniform tiles. Inside an
// expert: blocks of kGroupM (256) or kGroupM / 2 (512) M-tiles, N-tile-major
// inside a block.
template <int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_dma8_mixed_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDma8Lds];
  const int ntn = p.N / Dma8Shape<MODE, 256>::COLS;
  const int n_tiles = p.meta[0] * ntn;
  const int b = blockIdx.x;
  if (b >= n_tiles) return;
  const int j = xcd_chunked_tile(b, n_tiles);
  const int e = p.tile_e[j / ntn];
  const int ts = p.e_tstart[e], nm = p.e_ntiles[e];
  const int jj = j - ts * ntn;
  const int end = p.offsets[e + 1];
  TileInfo ti;
  ti.e = e;
  if (end - p.offsets[e] > 256) {
    constexpr int G = kGroupM / 2;
    const int nm2 = nm >> 1, ntn2 = 2 * ntn;
    const int mb = jj / (G * ntn2), rem = jj - mb * G * ntn2;
    const int gm = min(G, nm2 - mb * G);
    const int nt = rem / gm, m2 = mb * G + rem % gm;
    ti.row0 = p.tile_r[ts + 2 * m2];
    ti.rows = min(512, end - ti.row0);
    dma8_tile<MODE, 512>(p, ti, nt, smem);
  } else {
    ti.row0 = p.tile_r[ts];
    ti.rows = end - ti.row0;
    dma8_tile<MODE, 256>(p, ti, jj, smem);
  }
}

// ---------------------------------------------------------------- MXFP4 DMA variant
// Large batches with MXFP4 weights: the fp8 DMA variant's tiles, waves, tile
// order and half-stage ring, with the scaled fp8 x fp4 MFMA. A half-stage
// holds 64 bytes of every A row (chunk g of row r at position
// g ^ ((r >> 1) & 3)) and half of each of the 16 weight row blocks' 1 KB
// fragment blocks (lanes 0-31 or 32-63). Activation lane group a takes
// chunk a of both halves of its step (elements 16 a .. and 64 + 16 a ..),
// the order in which the instruction pairs it with whole 32-element weight
// lanes (see the streaming variant; the pairing is the same with the weights
// as the first operand, which gives the transposed output tile the epilogue
// expects). The E8M0 block scales of the tile's 16
// row blocks for four steps (4 KB) go to LDS by DMA at the first two
// half-stages of the previous four steps (double buffered); those extra
// loads only ever make the ring's wait counts stricter.
template <int MODE, int BM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_dma4_kernel(GemmArgs p) {
  constexpr int A_BYTES = BM * 64, B_BYTES = 16 * 512, STAGE = A_BYTES + B_BYTES;
  constexpr int SC_BYTES = 16 * 256;            // scales of 16 row blocks x 4 steps
  constexpr int NS0 = (150 * 1024 - 2 * SC_BYTES) / STAGE;
  constexpr int NS = NS0 > 8 ? 8 : NS0;         // 5 (BM 256) or 8 (BM 128) slots
  constexpr int AHEAD = NS - 2;
  constexpr int FM = BM / 32, FN = 4;
  constexpr int COLS = (MODE == 0) ? 128 : 256;
  constexpr int AI = BM / 128;
  static_assert(AHEAD >= 2, "ring too small");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE + 2 * SC_BYTES];
  uint8_t* scb = smem + NS * STAGE;

  const int ntn = p.N / COLS;
  const int n_tiles = p.meta[0] * ntn;
  const int b = blockIdx.x;
  if (b >= n_tiles) return;
  const int j = xcd_chunked_tile(b, n_tiles);
  const int e = p.tile_e[j / ntn];
  const int ts = p.e_tstart[e], nm = p.e_ntiles[e];
  const int jj = j - ts * ntn;
  const int mb = jj / (kGroupM * ntn), rem = jj - mb * kGroupM * ntn;
  const int gm = min(kGroupM, nm - mb * kGroupM);
  const int nt = rem / gm, mt = ts + mb * kGroupM + rem % gm;
  TileInfo ti;
  ti.e = e;
  ti.row0 = p.tile_r[mt];
  ti.rows = min(BM, p.offsets[e + 1] - ti.row0);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3, r = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N;
  const int n0 = nt * COLS;

  // A: as in the fp8 DMA variant.
  const uint8_t* asrc[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (wave * AI + i) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 1) & 3);
    const int ar = min(row, ti.rows - 1);
    const uint8_t* base = (MODE == 0) ? (const uint8_t*)p.a + (size_t)p.stok[ti.row0 + ar] * K
                                      : (const uint8_t*)p.a + (size_t)(ti.row0 + ar) * K;
    asrc[i] = base + chunk * 16;
  }
  // B: one instruction per wave and half-stage: lanes 0-31 load half h of
  // row block 2 wave, lanes 32-63 half h of row block 2 wave + 1.
  const uint8_t* bsrc;
  {
    const int rbk = wave * 2 + (lane >> 5);
    const uint8_t* W = (const uint8_t*)((MODE == 0 && rbk >= 8) ? p.w1 : p.w0);
    const int blk = (MODE == 0) ? (n0 >> 4) + (rbk & 7) : (n0 >> 4) + rbk;
    bsrc = W + (size_t)ti.e * N * (K / 2) + (size_t)blk * 8 * K + (lane & 31) * 16;
  }
  // Scales: in half-stage 8 q + i (i = 0, 1) wave w loads the dwords of steps
  // 4 (q + 1) .. + 3 of local row block 2 w + i (64 lanes x 4 bytes).
  const uint32_t* ssrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rbk = wave * 2 + i;
    const uint32_t* S = (const uint32_t*)((MODE == 0 && rbk >= 8) ? p.ws1 : p.ws0);
    const int blk = (MODE == 0) ? (n0 >> 4) + (rbk & 7) : (n0 >> 4) + rbk;
    ssrc[i] = S + ((size_t)ti.e * (N / 16) + blk) * (K / 512) * 64 + lane;
  }
  auto scale_dma = [&](int grp, int i) {  // step group grp of local row block 2 wave + i
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(ssrc[i] + (size_t)grp * 64,
                                     scb + (grp & 1) * SC_BYTES + (wave * 2 + i) * 256, 4, 0, 0);
#endif
  };
  auto issue = [&](int hs, auto al_c) {
    constexpr int AL = decltype(al_c)::value;
    uint8_t* st = smem + (hs % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < AL; ++i) dma16(asrc[i] + (size_t)hs * 64, st + (wave * AI + i) * 1024);
    dma16_nt(bsrc + (size_t)(hs >> 1) * 1024 + (hs & 1) * 512, st + A_BYTES + wave * 1024);
  };

  // Operand offsets: A chunk g of this lane's row (both halves of the step),
  // B: this lane's 16 bytes in half lane / 32 of its row block's block.
  const int half = lane >> 5;
  int aoff[FM], boff[FN], soff[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int row = wm * (BM / 2) + f * 16 + r;
    aoff[f] = row * 64 + ((g ^ ((row >> 1) & 3)) << 4);
  }
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int rbl = (MODE == 0) ? ((f < 2) ? wn * 2 + f : 8 + wn * 2 + (f - 2)) : wn * 4 + f;
    boff[f] = A_BYTES + rbl * 512 + (lane & 31) * 16;
    soff[f] = rbl * 256 + lane * 4;
  }
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nh = K / 64;  // a multiple of 8
  auto kloop = [&](auto nf_c, auto al_c) {
    constexpr int NF = decltype(nf_c)::value;
    constexpr int PER = decltype(al_c)::value + 1;  // A and B DMAs per half-stage
    scale_dma(0, 0);  // step group 0
    scale_dma(0, 1);
#pragma unroll
    for (int s0 = 0; s0 < AHEAD; ++s0)
      if (s0 < nh) issue(s0, al_c);
    for (int hs = 0; hs < nh; ++hs) {
      if (hs + AHEAD - 1 < nh)
        wait_vmcnt<(AHEAD - 1) * PER>();
      else
        wait_vmcnt<0>();
      barrier_only();
      asm volatile("" ::: "memory");
      if (hs + AHEAD < nh) issue(hs + AHEAD, al_c);
      // scales of the next step group, at the first two half-stages of a
      // group: the buffer they fill was last read by the previous group,
      // whose reads every wave retired before this barrier; they are read
      // from half-stage 8 (q + 1) + 1 on, whose wait retires them first
      if ((hs & 7) < 2 && ((hs >> 3) + 1) * 8 < nh) scale_dma((hs >> 3) + 1, hs & 7);
      if constexpr (NF > 0) {
        if (hs & 1) {
          const int s = hs >> 1;
          const uint8_t* st0 = smem + ((hs - 1) % NS) * STAGE;
          const uint8_t* st1 = smem + (hs % NS) * STAGE;
          const uint8_t* stb = half ? st1 : st0;
          const uint8_t* sc = scb + ((s >> 2) & 1) * SC_BYTES;
          i32x8 bfr[FN];
          int bsc[FN];
#pragma unroll
          for (int f = 0; f < FN; ++f) {
            const u32x4 v = ld16(stb + boff[f]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              bfr[f][i] = (int)v[i];
              bfr[f][4 + i] = 0;
            }
            bsc[f] = (int)((*reinterpret_cast<const uint32_t*>(sc + soff[f]) >> (8 * (s & 3))) & 0xffu);
          }
          // A fragment i + 1 is read while the MFMAs of fragment i execute
          u32x4 alo[NF], ahi[NF];
          alo[0] = ld16(st0 + aoff[0]);
          ahi[0] = ld16(st1 + aoff[0]);
#pragma unroll
          for (int i = 0; i < NF; ++i) {
            i32x8 a;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              a[q] = (int)alo[i][q];
              a[4 + q] = (int)ahi[i][q];
            }
#pragma unroll
            for (int jn = 0; jn < FN; ++jn) acc[i][jn] = mfma_fp4_fp8(bfr[jn], a, bsc[jn], acc[i][jn]);
            if (i + 1 < NF) {
              alo[i + 1] = ld16(st0 + aoff[i + 1]);
              ahi[i + 1] = ld16(st1 + aoff[i + 1]);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, FN - 2, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      wait_lgkmcnt0();
      asm volatile("" ::: "memory");
    }
  };
  const int need = min(FM, max(0, (ti.rows - wm * (BM / 2) + 15) >> 4));
  const int al = min(AI, max(0, (ti.rows - wave * AI * 16 + 15) >> 4));
  auto run = [&](auto nf_c) {
    if (al == 0)
      kloop(nf_c, std::integral_constant<int, 0>{});
    else if (al == 1)
      kloop(nf_c, std::integral_constant<int, 1>{});
    else
      kloop(nf_c, std::integral_constant<int, AI>{});
  };
  if (need == 0)
    run(std::integral_constant<int, 0>{});
  else if (need <= FM / 4)
    run(std::integral_constant<int, FM / 4>{});
  else if (need <= FM / 2)
    run(std::integral_constant<int, FM / 2>{});
  else
    run(std::integral_constant<int, FM>{});

  transposed_epilogue<MODE, true, FM, FN, true>(p, ti, acc, wm * (BM / 2), n0, wn, r, g);
}

// ---------------------------------------------------------------- launchers
int mtile_bound(const Shape& s, int BM) {
  const long long pairs = (long long)s.T * s.top_k;
  const long long active = pairs < s.E ? pairs : s.E;
  // mixed heights: 256-row slots, at most two more per expert than its rows need
  if (BM == kMixedBM) return (int)(2 * active + pairs / 256 + 1);
  return (int)(active + pairs / BM + 1);
}

bool use_stream_gemm(const Shape& s) {
  // Packed fp8 weights: the DMA variant streams them faster at every batch
  // size (at 64 tokens 6.3 TB/s against 5.6 for the register-streaming one).
  if (s.w_fp8 && !s.w_mx4 && s.w_packed) return false;
  // Otherwise up to about 16 rows per expert on average (12 for MXFP4) the
  // weights are streamed once per M-tile; beyond that the LDS-tiled variants
  // reuse them better.
  const long long rows = s.w_mx4 ? 12 : 16;
  return (long long)s.T * s.top_k <= rows * s.E;
}

int stream_bm(const Shape& s) {
  // Above 8 rows per expert on average a good part of the experts exceed 16
  // rows (at 16 on average, about 45% of them): 32-row tiles keep such an
  // expert to one M-tile, so its weights are streamed once.
  return (long long)s.T * s.top_k > 8LL * s.E ? 2 * kStreamBM : kStreamBM;
}

// Register-ring depth (k-steps in flight per wave) of the streaming kernels
// for FN fragments per wave and MR row blocks: 4 for waves of 2 fragments (the
// narrow workgroups of an expert shard, which would otherwise keep 4 KB in
// flight) and for the bf16 decode waves (8 fragments with one row block, 4
// with two: still two waves per SIMD); else 2, which keeps wider operands
// (fp8, fp32 tokens) at two waves per SIMD.
constexpr int stream_depth(int fn, int mr, bool bf16_ops) {
  return (fn == 2 || (bf16_ops && ((fn == 8 && mr == 1) || (fn == 4 && mr == 2)))) ? 4 : 2;
}

template <int MODE, typename AT, bool FP8, bool PACKED, int MR>
static void launch_stream_mr(dim3 grid, int fn, const GemmArgs& g, hipStream_t st) {
  constexpr bool B16 = !FP8 && std::is_same<AT, uint16_t>::value;
  if (fn == 8)
    gemm_stream_kernel<MODE, AT, FP8, PACKED, 8, stream_depth(8, MR, B16), MR><<<grid, 256, 0, st>>>(g);
  else if (fn == 4)
    gemm_stream_kernel<MODE, AT, FP8, PACKED, 4, stream_depth(4, MR, B16), MR><<<grid, 256, 0, st>>>(g);
  else
    gemm_stream_kernel<MODE, AT, FP8, PACKED, 2, stream_depth(2, MR, B16), MR><<<grid, 256, 0, st>>>(g);
}

// Output columns per workgroup: 4 waves x 16 x FN (down) or x 16 x FN/2
// (gate/up). FN = 8 where it divides N, else 4, else 2 (N is a multiple of 128).
template <int MODE, typename AT, bool FP8, bool PACKED>
static void launch_stream(const Shape& s, const GemmArgs& g, hipStream_t st) {
  const int per = (MODE == 0) ? 32 : 64;  // columns per workgroup per unit of FN
  int fn = (g.N % (8 * per) == 0) ? 8 : (g.N % (4 * per) == 0) ? 4 : 2;
  // Few experts running (an expert shard): narrower workgroups, so that
  // about 1024 stream weights at once (one M-tile per expert at decode).
  while (fn > 2 && (long long)s.n_run * (g.N / (fn * per)) < 1024) fn /= 2;
  const int bm = stream_bm(s);
  // Two row blocks: 4 fragments per wave. With fp8 operands (twice the
  // registers of bf16) 8 would leave one wave per SIMD; with bf16 tokens 4
  // fragments and a 4-deep ring stream 1% faster at 384 and 512 tokens.
  constexpr bool B16 = !FP8 && std::is_same<AT, uint16_t>::value;
  if ((FP8 || B16) && bm != kStreamBM && fn == 8) fn = 4;
  dim3 grid(mtile_bound(s, bm) * (g.N / (fn * per)));
  if (bm == kStreamBM)
    launch_stream_mr<MODE, AT, FP8, PACKED, 1>(grid, fn, g, st);
  else
    launch_stream_mr<MODE, AT, FP8, PACKED, 2>(grid, fn, g, st);
}

template <int MODE, typename AT, bool FP8, bool PACKED>
static void launch_tiled(const Shape& s, const GemmArgs& g, hipStream_t st) {
  dim3 grid(mtile_bound(s, kTiledBM) * (g.N / (MODE == 0 ? 64 : 128)));
  gemm_tiled_kernel<MODE, AT, FP8, PACKED><<<grid, 256, 0, st>>>(g);
}

int wide_bm(const Shape& s) {
  // An expert whose rows span two M-tiles has its weights read once per tile
  // (the second read hits L2 only when both tiles run in step). The DMA
  // variants (bf16 tokens, or fp8 weights) skip the matrix-core work of
  // fragments without live rows, so they take 256-row tiles once experts
  // average 96 rows; the register-staged variant (fp32 tokens, bf16 weights)
  // computes whole tiles and switches at 192. With a hidden size that is not
  // a multiple of 256 the down pass runs the 128-row tiled kernel (256-column
  // tiles do not divide it), and both passes walk one tile list: 128 rows.
  const long long pairs = (long long)s.T * s.top_k;
  const bool dma = s.w_fp8 || !s.x_f32;
  if (s.H % 256 != 0) return 128;
  return pairs >= (dma ? 96LL : 192LL) * s.E ? 256 : 128;
}

int forward_list_bm(const Shape& s) {
  if (use_stream_gemm(s)) return stream_bm(s);
  if (!s.w_packed) return kTiledBM;
  const int bm = wide_bm(s);
  // packed fp8 weights at 256-row tiles: 512-row tiles for experts beyond 256 rows
  if (bm == 256 && s.w_fp8 && !s.w_mx4) return kMixedBM;
  return bm;
}

template <int MODE, typename AT, bool FP8, int BM>
static void launch_wide_bm(const Shape& s, const GemmArgs& g, hipStream_t st) {
  // The grid is a bound on the active tile count, rounded up to a multiple of
  // the 8 XCDs; blocks past the active count exit at once.
  long long n = (long long)mtile_bound(s, BM) * (g.N / (MODE == 0 ? 128 : 256));
  n = (n + 7) & ~7LL;
  if constexpr (FP8)
    gemm_dma8_kernel<MODE, BM><<<(unsigned)n, 512, 0, st>>>(g);
  else if constexpr (std::is_same<AT, uint16_t>::value)
    gemm_dma_kernel<MODE, BM><<<(unsigned)n, 512, 0, st>>>(g);
  else
    gemm_wide_kernel<MODE, AT, FP8, BM><<<(unsigned)n, 512, 0, st>>>(g);
}

template <int MODE, typename AT, bool FP8>
static void launch_wide(const Shape& s, const GemmArgs& g, hipStream_t st) {
  const int lbm = forward_list_bm(s);
  if constexpr (FP8) {
    if (lbm == kMixedBM) {
      // one unit per (256-row slot, 256-row-tile N-tile); surplus units exit
      long long n = (long long)mtile_bound(s, kMixedBM) * (g.N / Dma8Shape<MODE, 256>::COLS);
      n = (n + 7) & ~7LL;
      gemm_dma8_mixed_kernel<MODE><<<(unsigned)n, 512, 0, st>>>(g);
      return;
    }
  }
  if (lbm == 256)
    launch_wide_bm<MODE, AT, FP8, 256>(s, g, st);
  else
    launch_wide_bm<MODE, AT, FP8, 128>(s, g, st);
}

template <int MODE, typename AT, bool FP8>
static void launch_variant(const Shape& s, const GemmArgs& g, hipStream_t st) {
  const bool stream = use_stream_gemm(s);
  if (s.w_packed) {
    if (stream)
      launch_stream<MODE, AT, FP8, true>(s, g, st);
    else if (g.N % (MODE == 0 ? 128 : 256) == 0)
      launch_wide<MODE, AT, FP8>(s, g, st);
    else  // down pass with hidden not a multiple of 256: 128-column tiles
      launch_tiled<MODE, AT, FP8, true>(s, g, st);
  } else {
    if (stream)
      launch_stream<MODE, AT, FP8, false>(s, g, st);
    else
      launch_tiled<MODE, AT, FP8, false>(s, g, st);
  }
}

// MXFP4 weights: the streaming variant for decode-sized batches (hidden and
// intermediate are multiples of 512, so 8 fragments per wave always divide),
// the DMA variant beyond.
template <int MODE>
static void launch_mx4(const Shape& s, const GemmArgs& g, hipStream_t st) {
  if (use_stream_gemm(s)) {
    // 8 fragments per wave with one row block (register ring 4 k-steps deep),
    // 4 with two (ring depth 2, two waves per SIMD)
    const int bm = stream_bm(s);
    if (bm == kStreamBM) {
      constexpr int FN = 8, per = (MODE == 0) ? 4 * 16 * FN / 2 : 4 * 16 * FN;
      dim3 grid(mtile_bound(s, bm) * (g.N / per));
      gemm_stream4_kernel<MODE, FN, 4, 1><<<grid, 256, 0, st>>>(g);
    } else {
      constexpr int FN = 4, per = (MODE == 0) ? 4 * 16 * FN / 2 : 4 * 16 * FN;
      dim3 grid(mtile_bound(s, bm) * (g.N / per));
      gemm_stream4_kernel<MODE, FN, 2, 2><<<grid, 256, 0, st>>>(g);
    }
    return;
  }
  const int BM = wide_bm(s);
  long long n = (long long)mtile_bound(s, BM) * (g.N / (MODE == 0 ? 128 : 256));
  n = (n + 7) & ~7LL;
  if (BM == 256)
    gemm_dma4_kernel<MODE, 256><<<(unsigned)n, 512, 0, st>>>(g);
  else
    gemm_dma4_kernel<MODE, 128><<<(unsigned)n, 512, 0, st>>>(g);
}

hipError_t launch_gateup(const Shape& s, const GemmArgs& g, hipStream_t st) {
  if (s.w_mx4)
    launch_mx4<0>(s, g, st);
  else if (s.w_fp8)
    launch_variant<0, uint8_t, true>(s, g, st);
  else if (s.x_f32)
    launch_variant<0, float, false>(s, g, st);
  else
    launch_variant<0, uint16_t, false>(s, g, st);
  return hipGetLastError();
}

template <int MODE>
static void launch_backward_bm(const Shape& s, int BM, const GemmArgs& g, hipStream_t st) {
  long long n = (long long)mtile_bound(s, BM) * (g.N / (mode_paired(MODE) ? 128 : 256));
  n = (n + 7) & ~7LL;
  if (BM == 256)
    gemm_dma_kernel<MODE, 256><<<(unsigned)n, 512, 0, st>>>(g);
  else
    gemm_dma_kernel<MODE, 128><<<(unsigned)n, 512, 0, st>>>(g);
}

hipError_t launch_backward_gemm(int mode, const Shape& s, int BM, const GemmArgs& g,
                                hipStream_t st) {
  if (mode == 2)
    launch_backward_bm<2>(s, BM, g, st);
  else if (mode == 3)
    launch_backward_bm<3>(s, BM, g, st);
  else if (mode == 4)
    launch_backward_bm<4>(s, BM, g, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_down(const Shape& s, const GemmArgs& g, hipStream_t st) {
  if (s.w_mx4)
    launch_mx4<1>(s, g, st);
  else if (s.w_fp8)
    launch_variant<1, uint8_t, true>(s, g, st);
  else
    launch_variant<1, uint16_t, false>(s, g, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- weight packing
// Row-major [rows, cols] matrices (cols = the reduction) to the MFMA fragment
// layout: one block per (16-row block, k-step) holding the 64 lanes' operand
// bytes in lane order (lane l: row l % 16, k-step bytes (l / 16) * LB ..).
// SB = bytes of one k-step of one row (64 for bf16, 128 for fp8), LB = SB / 4.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src,
                                                   uint8_t* __restrict__ dst, long long chunks,
                                                   long long mat_bytes, int row_bytes, int SB) {
  const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const long long o = c * 16;
  const long long e = o / mat_bytes, rem = o % mat_bytes;
  const int BLK = 16 * SB, LB = SB / 4;
  const long long bidx = rem / BLK;
  const int w = (int)(rem % BLK);
  const int steps = row_bytes / SB;
  const long long rb = bidx / steps;
  const int st = (int)(bidx % steps);
  const int lane = w / LB, j = w % LB;
  const long long row = rb * 16 + (lane & 15);
  const long long kb = (long long)st * SB + (lane >> 4) * LB + j;
  st16(dst + o, ld16(src + e * mat_bytes + row * row_bytes + kb));
}

hipError_t launch_pack_bytes(const void* src, void* dst, int E, int rows, int row_bytes, int SB,
                             hipStream_t st) {
  const long long mat = (long long)rows * row_bytes;
  const long long chunks = (long long)E * mat / 16;
  const long long blocks = (chunks + 255) / 256;
  pack_kernel<<<(unsigned)blocks, 256, 0, st>>>((const uint8_t*)src, (uint8_t*)dst, chunks, mat,
                                                row_bytes, SB);
  return hipGetLastError();
}

// MXFP4 scale bytes, row-major [E, rows, cols / 32] -> packed: the dword of
// (row block rb, step group q, lane l) holds, in byte j, the scale of row
// 16 rb + l % 16 and column block 16 q + 4 j + l / 16 (step 4 q + j).
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* __restrict__ src,
                                                             uint32_t* __restrict__ dst,
                                                             long long dwords, int rows, int cols) {
  const long long d = (long long)blockIdx.x * 256 + threadIdx.x;
  if (d >= dwords) return;
  const int nb = cols / 32, nq = cols / 512;
  const int lane = (int)(d & 63);
  long long t = d >> 6;
  const int q = (int)(t % nq);
  t /= nq;
  const int rb = (int)(t % (rows / 16));
  const long long e = t / (rows / 16);
  const long long row = (long long)rb * 16 + (lane & 15);
  const uint8_t* sr = src + (e * rows + row) * nb + 16 * q + (lane >> 4);
  dst[d] = (uint32_t)sr[0] | ((uint32_t)sr[4] << 8) | ((uint32_t)sr[8] << 16) |
           ((uint32_t)sr[12] << 24);
}

hipError_t launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, int E, int rows, int cols,
                                 hipStream_t st) {
  const long long dwords = (long long)E * rows * (cols / 32) / 4;
  pack_mx_scales_kernel<<<(unsigned)((dwords + 255) / 256), 256, 0, st>>>(src, (uint32_t*)dst, dwords,
                                                                          rows, cols);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, void* dst, int E, int rows, int cols, int fp8,
                       hipStream_t st) {
  const int esz = fp8 ? 1 : 2;
  const long long mat = (long long)rows * cols * esz;
  const long long chunks = (long long)E * mat / 16;
  const long long blocks = (chunks + 255) / 256;
  pack_kernel<<<(unsigned)blocks, 256, 0, st>>>((const uint8_t*)src, (uint8_t*)dst, chunks, mat,
                                                cols * esz, fp8 ? 128 : 64);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine
// out[t] = sum over slots j (ascending) of y_perm[inv[t, j]], in fp32; the
// rows already carry rsf * w. One thread per 8 output values. Every y row is
// read once, so with the non-temporal hint.
template <int OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ inv, int T,
                                                      int k, int H, void* __restrict__ out) {
  const int vpr = H / 8;
  const long long v = (long long)blockIdx.x * 256 + threadIdx.x;
  if (v >= (long long)T * vpr) return;
  const int t = (int)(v / vpr), c = (int)(v % vpr);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll 4
  for (int j = 0; j < k; ++j) {
    const int pos = inv[(size_t)t * k + j];
    const u32x4 q = ld16_nt(y + (size_t)pos * H + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_bits_to_f32(q[i] & 0xffffu);
      acc[2 * i + 1] += bf16_bits_to_f32(q[i] >> 16);
    }
  }
  if (OUT_F32) {
    float* o = (float*)out + (size_t)t * H + c * 8;
    st16(o, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                  __float_as_uint(acc[3])});
    st16(o + 4, u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]),
                      __float_as_uint(acc[7])});
  } else {
    uint16_t* o = (uint16_t*)out + (size_t)t * H + c * 8;
    st16(o, u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])});
  }
}

hipError_t launch_combine(const void* y, const int32_t* inv, int T, int k, int H, int out_f32,
                          void* out, hipStream_t st) {
  const long long n = (long long)T * (H / 8);
  const int blocks = (int)((n + 255) / 256);
  if (out_f32)
    combine_kernel<1><<<blocks, 256, 0, st>>>((const uint16_t*)y, inv, T, k, H, out);
  else
    combine_kernel<0><<<blocks, 256, 0, st>>>((const uint16_t*)y, inv, T, k, H, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine + residual step
// One workgroup per token. The token's MoE output v (the fp32 sum over its
// slots, as in combine_kernel) stays in registers, RMS over the hidden
// dimension by a workgroup reduction, then
//   out = keep * stream_in + add * (v * rstd * gain),  rstd = 1 / sqrt(mean v^2 + eps).
// Each thread reads its own stream_in values before writing them, so
// stream_out may be the same memory as stream_in. 1024 threads per token (a
// decode batch has few tokens: the width keeps enough loads in flight);
// kResidualChunks chunks of 8 per thread cover H <= 1024 * 8 * kResidualChunks.
constexpr int kResidualThreads = 1024;
constexpr int kResidualChunks = kResidualMaxH / (kResidualThreads * 8);

template <typename XT>
__global__ __launch_bounds__(kResidualThreads) void combine_residual_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ inv, int k, int H,
    const XT* stream_in, const float* __restrict__ gain, float eps, float keep, float add,
    XT* stream_out) {
  constexpr int kWaves = kResidualThreads / 64;
  __shared__ float red[kWaves];
  const int t = blockIdx.x, vpr = H / 8;
  const int32_t* slots = inv + (size_t)t * k;
  float acc[kResidualChunks][8];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < kResidualChunks; ++u) {
    const int c = threadIdx.x + kResidualThreads * u;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
    if (c < vpr) {
#pragma unroll 4
      for (int j = 0; j < k; ++j) {
        const u32x4 q = ld16_nt(y + (size_t)slots[j] * H + c * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[u][2 * i] += bf16_bits_to_f32(q[i] & 0xffffu);
          acc[u][2 * i + 1] += bf16_bits_to_f32(q[i] >> 16);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += acc[u][i] * acc[u][i];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) tot += red[i];
  const float mean = tot / (float)H;
  const float rstd = 1.0f / sqrtf(mean + eps);
  const float scale = add * rstd;
  const XT* srow = stream_in + (size_t)t * H;
  XT* orow = stream_out + (size_t)t * H;
#pragma unroll
  for (int u = 0; u < kResidualChunks; ++u) {
    const int c = threadIdx.x + kResidualThreads * u;
    if (c < vpr) {
      ALoad16<XT> sv;
      sv.load(srow + c * 8);
      float s[8], o[8];
      sv.floats(s);
      const u32x4 g0 = ld16(gain + c * 8), g1 = ld16(gain + c * 8 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] = keep * s[i] + scale * acc[u][i] * __uint_as_float(g0[i]);
        o[4 + i] = keep * s[4 + i] + scale * acc[u][4 + i] * __uint_as_float(g1[i]);
      }
      if constexpr (sizeof(XT) == 4) {
        st16(orow + c * 8, u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]),
                                 __float_as_uint(o[2]), __float_as_uint(o[3])});
        st16(orow + c * 8 + 4, u32x4{__float_as_uint(o[4]), __float_as_uint(o[5]),
                                     __float_as_uint(o[6]), __float_as_uint(o[7])});
      } else {
        st16(orow + c * 8, u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                 pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])});
      }
    }
  }
}

hipError_t launch_combine_residual(const void* y, const int32_t* inv, int T, int k, int H,
                                   int x_f32, const void* stream_in, const float* gain, float eps,
                                   float keep, float add, void* stream_out, hipStream_t st) {
  if (H > kResidualMaxH || H % 8) return hipErrorInvalidValue;
  if (x_f32)
    combine_residual_kernel<float><<<T, kResidualThreads, 0, st>>>((const uint16_t*)y, inv, k, H,
                                                      (const float*)stream_in, gain, eps, keep,
                                                      add, (float*)stream_out);
  else
    combine_residual_kernel<uint16_t><<<T, kResidualThreads, 0, st>>>((const uint16_t*)y, inv, k, H,
                                                         (const uint16_t*)stream_in, gain, eps,
                                                         keep, add, (uint16_t*)stream_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fp8 quantisation
// Per-row E4M3 quantisation: amax = max |v|; scale = amax / 448 (1 if amax is
// 0); code = e4m3(v * (448 / amax)), all correctly rounded fp32 operations.

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One workgroup per token; also clears the token's top_k entries of the
// running |h| maxima used by the gate/up pass (rows t*k .. t*k+k-1 of the
// sorted order: together the T workgroups clear all T*k rows).
template <typename XT>
__global__ __launch_bounds__(256) void quant_x_kernel(const XT* __restrict__ x, int H,
                                                      uint8_t* __restrict__ xq,
                                                      float* __restrict__ xs,
                                                      uint32_t* __restrict__ hamax, int k) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const XT* row = x + (size_t)t * H;
  float m = 0.f;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    ALoad16<XT> v;
    v.load(row + c);
    float f[8];
    v.floats(f);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  }
  const float amax = block_max(m, red);
  const float inv = amax > 0.f ? 448.0f / amax : 0.f;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    ALoad16<XT> v;
    v.load(row + c);
    float f[8];
    v.floats(f);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= f32_to_e4m3(f[i] * inv) << (8 * (i & 3));
    *reinterpret_cast<u32x2*>(xq + (size_t)t * H + c) = u32x2{w[0], w[1]};
  }
  if (threadIdx.x == 0) xs[t] = amax > 0.f ? amax / 448.0f : 1.0f;
  if (threadIdx.x < k) hamax[(size_t)t * k + threadIdx.x] = 0u;
}

// One workgroup per sorted row of h.
__global__ __launch_bounds__(256) void quant_h_kernel(const uint16_t* __restrict__ hb,
                                                      const uint32_t* __restrict__ hamax, int I,
                                                      uint8_t* __restrict__ hq,
                                                      float* __restrict__ hs) {
  const size_t row = blockIdx.x;
  const float amax = __uint_as_float(hamax[row]);
  const float inv = amax > 0.f ? 448.0f / amax : 0.f;
  for (int c = threadIdx.x * 8; c < I; c += 256 * 8) {
    const u32x4 v = ld16_nt(hb + row * I + c);  // h is read once
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = (v[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      w[i >> 2] |= f32_to_e4m3(bf16_bits_to_f32(bits) * inv) << (8 * (i & 3));
    }
    *reinterpret_cast<u32x2*>(hq + row * I + c) = u32x2{w[0], w[1]};
  }
  if (threadIdx.x == 0) hs[row] = amax > 0.f ? amax / 448.0f : 1.0f;
}

hipError_t launch_quant_x(const void* x, int x_f32, int T, int H, int k, uint8_t* xq, float* xs,
                          uint32_t* hamax, hipStream_t st) {
  if (x_f32)
    quant_x_kernel<float><<<T, 256, 0, st>>>((const float*)x, H, xq, xs, hamax, k);
  else
    quant_x_kernel<uint16_t><<<T, 256, 0, st>>>((const uint16_t*)x, H, xq, xs, hamax, k);
  return hipGetLastError();
}

hipError_t launch_quant_h(const uint16_t* hb, const uint32_t* hamax, int rows, int I, uint8_t* hq,
                          float* hs, hipStream_t st) {
  quant_h_kernel<<<rows, 256, 0, st>>>(hb, hamax, I, hq, hs);
  return hipGetLastError();
}

}  // namespace beam
