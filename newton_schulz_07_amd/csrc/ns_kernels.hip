// ns_kernels.hip - HIP kernels of the Newton–Schulz orthogonalization for
// gfx950 (CDNA4): a two-pass Frobenius normalisation and one LDS-tiled MFMA
// kernel template that runs the three products of each step.
//
// Method (prime-rl PR #3873, "Summary" item 1; Megatron-LM PR #6381,
// "Summary"): per step A = X Xᵀ and B = b A + c A A are symmetric, so only
// lower-triangle tiles are computed and each is stored twice (mirror); the
// update X' = a X + B X is one product with the a X term folded into the
// fp32 epilogue.  A and C = a I + B are held as a zero-diagonal matrix in the
// storage dtype plus an fp32 diagonal vector, so their dominant diagonals
// never pass through bf16 (the page credits fp32 epilogue arithmetic for the
// symmetric path's accuracy; this placement extends that to the diagonals).
//
// Both operands of every product are staged in LDS as rows of K-contiguous
// 16-byte chunks, so one inner loop serves all products:
//   Gram, rows <= cols: P = Q = X rows              (K-contiguous in HBM)
//   Gram, rows >  cols: P = Q = X columns           (transposed on load)
//   poly:               P = Q = O_A rows            (A symmetric: A A = A Aᵀ)
//   update, wide:       P = O_C rows, Q = X columns (transposed on load)
//   update, tall:       P = X rows,   Q = O_C rows  (C symmetric)
// Tall matrices are never transposed in HBM: their Gram side is the column
// side, and X' = X C replaces the transpose-update-transpose.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ns_kernels.h"
#include "ns_layout.h"

namespace ns {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct Elem;
template <> struct Elem<bf16> { static constexpr int kChunk = 8; };
template <> struct Elem<float> { static constexpr int kChunk = 4; };

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// 16-byte chunk of operand values -> one MFMA step of the 32x32 block.
// bf16: the chunk is the 8-element k slice of v_mfma_f32_32x32x16_bf16.
// fp32: the chunk is 4 k values, one per v_mfma_f32_32x32x2_f32; A and B use
// the same k assignment, so the sum is the same product.
__device__ __forceinline__ void mfma_chunk(f32x16& acc, uint4 a, uint4 b, bf16) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_chunk(f32x16& acc, uint4 a, uint4 b, float) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Transpose an EPC x EPC block held as EPC k-rows of 16 bytes (EPC values
// along i) into EPC chunks of EPC values along k (one per i).
__device__ __forceinline__ void transpose_block(const uint4* in, uint4* out, bf16) {
  // dword d of k-row kk holds i = 2d (low half) and i = 2d+1 (high half).
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) w[kk] = u4get(in[kk], d);
    // v_perm_b32(hi, lo, sel): bytes 0-3 come from lo, 4-7 from hi.
    out[2 * d] = make_uint4(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u),
                            __builtin_amdgcn_perm(w[3], w[2], 0x05040100u),
                            __builtin_amdgcn_perm(w[5], w[4], 0x05040100u),
                            __builtin_amdgcn_perm(w[7], w[6], 0x05040100u));
    out[2 * d + 1] = make_uint4(__builtin_amdgcn_perm(w[1], w[0], 0x07060302u),
                                __builtin_amdgcn_perm(w[3], w[2], 0x07060302u),
                                __builtin_amdgcn_perm(w[5], w[4], 0x07060302u),
                                __builtin_amdgcn_perm(w[7], w[6], 0x07060302u));
  }
}
__device__ __forceinline__ void transpose_block(const uint4* in, uint4* out, float) {
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
    out[ii] = make_uint4(u4get(in[0], ii), u4get(in[1], ii), u4get(in[2], ii), u4get(in[3], ii));
}

// ----------------------------------------------------------------- loaders

template <typename T, int LAYOUT, int R, int NT> struct OperandLoader;

template <typename T, int R, int NT> struct OperandLoader<T, KCONT, R, NT> {
  static constexpr int EPC = Elem<T>::kChunk;
  static constexpr int NCH = R * 8;                   // chunks per stage
  static constexpr int ITER = (NCH + NT - 1) / NT;
  static constexpr int REGS = ITER;
  __device__ __forceinline__ static void load(const T* base, int ld, int r0, int rmax, int k0,
                                              int kmax, uint4* regs, int tid) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int qd = tid + it * NT;
      const KcontSrc s = kcont_src(qd);
      const int gi = r0 + s.row, gk = k0 + s.ch * EPC;
      const bool ok = (NCH % NT == 0 || qd < NCH) && gi < rmax && gk < kmax;
      regs[it] = ok ? ldg16(base + (size_t)gi * ld + gk) : zero4();
    }
  }
  __device__ __forceinline__ static void store(uint4* lds, const uint4* regs, int tid) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int qd = tid + it * NT;
      if (NCH % NT == 0 || qd < NCH) {
        const KcontSrc s = kcont_src(qd);
        lds[lds_swz(s.row, s.ch)] = regs[it];
      }
    }
  }
};

template <typename T, int R, int NT> struct OperandLoader<T, MCONT, R, NT> {
  static constexpr int EPC = Elem<T>::kChunk;
  static constexpr int IB = R / EPC;                  // i-blocks per stage
  static constexpr int NBLK = IB * 8;                 // 8 k-blocks (BK = 8 EPC)
  static constexpr int ITER = (NBLK + NT - 1) / NT;
  static constexpr int REGS = ITER * EPC;
  __device__ __forceinline__ static void load(const T* base, int ld, int r0, int rmax, int k0,
                                              int kmax, uint4* regs, int tid) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int qd = tid + it * NT;
      const McontSrc s = mcont_src(qd, IB);
      const int gi = r0 + s.ib * EPC;
      const bool blk = (NBLK % NT == 0 || qd < NBLK) && gi < rmax;
#pragma unroll
      for (int kk = 0; kk < EPC; ++kk) {
        const int gk = k0 + s.kb * EPC + kk;
        regs[it * EPC + kk] = (blk && gk < kmax) ? ldg16(base + (size_t)gk * ld + gi) : zero4();
      }
    }
  }
  __device__ __forceinline__ static void store(uint4* lds, const uint4* regs, int tid) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int qd = tid + it * NT;
      if (NBLK % NT == 0 || qd < NBLK) {
        const McontSrc s = mcont_src(qd, IB);
        uint4 t[EPC];
        transpose_block(regs + it * EPC, t, T());
#pragma unroll
        for (int ii = 0; ii < EPC; ++ii) lds[lds_swz(s.ib * EPC + ii, s.kb)] = t[ii];
      }
    }
  }
};

// ------------------------------------------------------------- MFMA kernel

template <typename T, int BM, int BN, int WM, int WN, int PL, int QL, int MODE>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(const GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int EPC = Elem<T>::kChunk;
  constexpr int BK = 8 * EPC;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int SM = WTM / 32, SN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(!mode_is_tri(MODE) || BM == BN, "triangle modes need square tiles");
  using LP = OperandLoader<T, PL, BM, NT>;
  using LQ = OperandLoader<T, QL, BN, NT>;

  __shared__ uint4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = lin / g.tiles_per_slice;
  const int q = lin - slice * g.tiles_per_slice;
  int ti, tj;
  if (mode_is_tri(MODE)) tri_decode(q, ti, tj);
  else rect_decode(q, g.tiles_m, g.tiles_n, ti, tj);
  const int i0 = ti * BM, j0 = tj * BN;

  const T* P = reinterpret_cast<const T*>(g.P) + (size_t)slice * g.p_bs;
  const T* Q = reinterpret_cast<const T*>(g.Q) + (size_t)slice * g.q_bs;

  f32x16 acc[SM][SN];
#pragma unroll
  for (int a = 0; a < SM; ++a)
#pragma unroll
    for (int b = 0; b < SN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  uint4 pr[LP::REGS], qr[LQ::REGS];
  const int nk = (g.K + BK - 1) / BK;

  LP::load(P, g.ldp, i0, g.M, 0, g.K, pr, tid);
  LQ::load(Q, g.ldq, j0, g.N, 0, g.K, qr, tid);
  LP::store(lds[0], pr, tid);
  LQ::store(lds[0] + BM * 8, qr, tid);
  __syncthreads();

  const int half = lane >> 5, l32 = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      LP::load(P, g.ldp, i0, g.M, (kt + 1) * BK, g.K, pr, tid);
      LQ::load(Q, g.ldq, j0, g.N, (kt + 1) * BK, g.K, qr, tid);
    }
    const uint4* Ps = lds[cur];
    const uint4* Qs = lds[cur] + BM * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + half;
      uint4 af[SM], bq[SN];
#pragma unroll
      for (int a = 0; a < SM; ++a) af[a] = Ps[lds_swz(wm * WTM + a * 32 + l32, ch)];
#pragma unroll
      for (int b = 0; b < SN; ++b) bq[b] = Qs[lds_swz(wn * WTN + b * 32 + l32, ch)];
#pragma unroll
      for (int a = 0; a < SM; ++a)
#pragma unroll
        for (int b = 0; b < SN; ++b) mfma_chunk(acc[a][b], af[a], bq[b], T());
    }
    if (more) {
      LP::store(lds[cur ^ 1], pr, tid);
      LQ::store(lds[cur ^ 1] + BM * 8, qr, tid);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  T* O = reinterpret_cast<T*>(g.out) + (size_t)slice * g.o_bs;
  const T* E = reinterpret_cast<const T*>(g.E) + (size_t)slice * g.e_bs;
  const float* din = g.d_in + (size_t)slice * g.d_bs;
  float* dout = g.d_out + (size_t)slice * g.d_bs;
  const bool diag_tile = mode_is_tri(MODE) && ti == tj;

#pragma unroll
  for (int a = 0; a < SM; ++a)
#pragma unroll
    for (int b = 0; b < SN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + wm * WTM + a * 32 + acc_row(r, lane);
        const int col = j0 + wn * WTN + b * 32 + acc_col(lane);
        if (row >= g.M || col >= g.N) continue;
        const float v = acc[a][b][r];
        if (MODE == MODE_GRAM || MODE == MODE_POLY) {
          if (diag_tile && row < col) continue;  // written by the mirror
          if (row == col) {
            if (MODE == MODE_GRAM) {
              dout[row] = v;
            } else {
              const float d = din[row];
              dout[row] = g.ca + g.cb * d + g.cc * (v + d * d);
            }
            O[(size_t)row * g.ldo + col] = from_f32<T>(0.0f);
          } else {
            float w = v;
            if (MODE == MODE_POLY) {
              const float o = to_f32(E[(size_t)row * g.lde + col]);
              w = g.cb * o + g.cc * (v + (din[row] + din[col]) * o);
            }
            const T t = from_f32<T>(w);
            O[(size_t)row * g.ldo + col] = t;
            O[(size_t)col * g.ldo + row] = t;
          }
        } else {
          const float d = (MODE == MODE_UPD_ROW) ? din[row] : din[col];
          const float x = to_f32(E[(size_t)row * g.lde + col]);
          O[(size_t)row * g.ldo + col] = from_f32<T>(v + d * x);
        }
      }
}

// --------------------------------------------------------- normalisation

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float sumsq16(uint4 u, bf16) {
  float s = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = u4get(u, d);
    const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}
__device__ __forceinline__ float sumsq16(uint4 u, float) {
  float s = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float f = __uint_as_float(u4get(u, d));
    s = fmaf(f, f, s);
  }
  return s;
}

__device__ __forceinline__ uint4 scale16(uint4 u, float inv, bf16) {
  uint32_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = u4get(u, d);
    const bf16 lo = (bf16)(__uint_as_float(w << 16) * inv);
    const bf16 hi = (bf16)(__uint_as_float(w & 0xffff0000u) * inv);
    o[d] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
__device__ __forceinline__ uint4 scale16(uint4 u, float inv, float) {
  return make_uint4(__float_as_uint(__uint_as_float(u.x) * inv), __float_as_uint(__uint_as_float(u.y) * inv),
                    __float_as_uint(__uint_as_float(u.z) * inv), __float_as_uint(__uint_as_float(u.w) * inv));
}

constexpr int kNormThreads = 256;

// Pass 1: partial sums of squares, one per (chunk, slice) block, fixed order.
template <typename T>
__global__ __launch_bounds__(kNormThreads) void sumsq_kernel(const NormArgs g) {
  __shared__ float red[kNormThreads / 64];
  const int slice = blockIdx.y, chunk = blockIdx.x;
  const uint4* xv = reinterpret_cast<const uint4*>(g.x) + (size_t)slice * g.slice_vecs;
  const long long v0 = (long long)chunk * g.chunk_vecs;
  const long long v1 = (v0 + g.chunk_vecs < g.slice_vecs) ? v0 + g.chunk_vecs : g.slice_vecs;
  float s = 0.0f;
  for (long long v = v0 + threadIdx.x; v < v1; v += kNormThreads) s += sumsq16(xv[v], T());
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kNormThreads / 64; ++w) t += red[w];
    g.partials[(size_t)slice * g.chunks + chunk] = t;
  }
}

// Pass 2: every block sums its slice's partials (same order in every block),
// then writes x / (sqrt(sum) + eps) in the storage dtype.
template <typename T>
__global__ __launch_bounds__(kNormThreads) void scale_kernel(const NormArgs g) {
  __shared__ float s_inv;
  const int slice = blockIdx.y, chunk = blockIdx.x;
  if (threadIdx.x < 64) {
    float s = 0.0f;
    for (int i = threadIdx.x; i < g.chunks; i += 64) s += g.partials[(size_t)slice * g.chunks + i];
    s = wave_sum(s);
    if (threadIdx.x == 0) {
      const float nrm = sqrtf(s);
      s_inv = 1.0f / (nrm + g.eps);
      if (g.norms != nullptr && chunk == 0) g.norms[slice] = nrm;
    }
  }
  __syncthreads();
  const float inv = s_inv;
  const uint4* xv = reinterpret_cast<const uint4*>(g.x) + (size_t)slice * g.slice_vecs;
  uint4* yv = reinterpret_cast<uint4*>(g.y) + (size_t)slice * g.slice_vecs;
  const long long v0 = (long long)chunk * g.chunk_vecs;
  const long long v1 = (v0 + g.chunk_vecs < g.slice_vecs) ? v0 + g.chunk_vecs : g.slice_vecs;
  for (long long v = v0 + threadIdx.x; v < v1; v += kNormThreads) yv[v] = scale16(xv[v], inv, T());
}

// ------------------------------------------------------------- launchers

template <typename T, int BM, int BN, int WM, int WN, int PL, int QL, int MODE>
static hipError_t launch_gemm_t(const GemmArgs& g, hipStream_t st) {
  const int total = g.tiles_per_slice * g.batch;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, PL, QL, MODE>), dim3(total), dim3(WM * WN * 64),
                     0, st, g);
  return hipGetLastError();
}

template <typename T, int PL, int QL, int MODE>
static hipError_t dispatch_tile(const GemmArgs& g, hipStream_t st) {
  constexpr TileCfg t = std::is_same<T, bf16>::value ? kTileBf16 : kTileF32;
  return launch_gemm_t<T, t.bm, t.bn, t.wm, t.wn, PL, QL, MODE>(g, st);
}

template <typename T>
static hipError_t dispatch_mode(int mode, int pl, int ql, const GemmArgs& g, hipStream_t st) {
  if (mode == MODE_GRAM && pl == KCONT) return dispatch_tile<T, KCONT, KCONT, MODE_GRAM>(g, st);
  if (mode == MODE_GRAM && pl == MCONT) return dispatch_tile<T, MCONT, MCONT, MODE_GRAM>(g, st);
  if (mode == MODE_POLY) return dispatch_tile<T, KCONT, KCONT, MODE_POLY>(g, st);
  if (mode == MODE_UPD_ROW) return dispatch_tile<T, KCONT, MCONT, MODE_UPD_ROW>(g, st);
  if (mode == MODE_UPD_COL) return dispatch_tile<T, KCONT, KCONT, MODE_UPD_COL>(g, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int dtype, int mode, int p_layout, int q_layout, const GemmArgs& g,
                       hipStream_t st) {
  if (dtype == 1) return dispatch_mode<bf16>(mode, p_layout, q_layout, g, st);
  return dispatch_mode<float>(mode, p_layout, q_layout, g, st);
}

hipError_t launch_sumsq(int dtype, const NormArgs& g, int batch, hipStream_t st) {
  dim3 grid(g.chunks, batch);
  if (dtype == 1) hipLaunchKernelGGL(sumsq_kernel<bf16>, grid, dim3(kNormThreads), 0, st, g);
  else hipLaunchKernelGGL(sumsq_kernel<float>, grid, dim3(kNormThreads), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_scale(int dtype, const NormArgs& g, int batch, hipStream_t st) {
  dim3 grid(g.chunks, batch);
  if (dtype == 1) hipLaunchKernelGGL(scale_kernel<bf16>, grid, dim3(kNormThreads), 0, st, g);
  else hipLaunchKernelGGL(scale_kernel<float>, grid, dim3(kNormThreads), 0, st, g);
  return hipGetLastError();
}

}  // namespace ns
