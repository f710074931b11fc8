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
// The iterate is kept in HBM only in the input's orientation.  An operand is
// read either as K-contiguous rows (staged as chunks along k) or, where the
// reduction runs down the columns of the stored matrix, in its natural layout
// (staged as k rows and read back transposed with ds_read_b64_tr_b16):
//   Gram, rows <= cols: P = Q = rows of X                 (K-contiguous)
//   Gram, rows >  cols: P = Q = columns of X              (natural layout)
//   poly:               P = Q = rows of O_A  (A symmetric: A A = A Aᵀ)
//   update, wide:       P = rows of O_C, Q = columns of X (X' = C X)
//   update, tall:       P = rows of X,   Q = rows of O_C  (X' = X C)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "ns_kernels.h"
#include "ns_layout.h"
#include "ns_plan.h"

#ifndef NS_FRAG_BARRIER
#define NS_FRAG_BARRIER 1
#endif



namespace ns {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct Elem;
template <> struct Elem<bf16> { static constexpr int kChunk = 8; };
template <> struct Elem<float> { static constexpr int kChunk = 4; };

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)hi) << 16);
}

// 4 consecutive elements of type T <-> 4 floats
template <typename T> struct Quad;
template <> struct Quad<bf16> {
  typedef uint2 Raw;  // 8 bytes
  __device__ __forceinline__ static void unpack(Raw r, float* f) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
  }
  __device__ __forceinline__ static Raw pack(const float* f) {
    return make_uint2(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]));
  }
};
template <> struct Quad<float> {
  typedef uint4 Raw;  // 16 bytes
  __device__ __forceinline__ static void unpack(Raw r, float* f) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
  __device__ __forceinline__ static Raw pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

// 16-byte chunks of operand values -> one MFMA step of a 32x32 block.
// bf16: the chunk is the 8-element k slice of v_mfma_f32_32x32x16_bf16.
// fp32: the chunk is 4 k values, one per v_mfma_f32_32x32x2_f32; both
// operands use the same k assignment, so the sum is the same product.
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

// ------------------------------------------------------------- MFMA kernel

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor (gfx9 V#) over `bytes` bytes at `base`, stride 0: a load
// at an offset >= bytes returns zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  i32x4 r = {(int)(a & 0xffffffffu), (int)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
  return r;
}

// 16 bytes per lane from buffer offset voff into LDS at m0 + 16 * lane
// (buffer_load_dwordx4 ... lds).  Issued through asm so that the compiler,
// which cannot tell ring slots apart, does not wait for these loads before
// every LDS read; the kernel waits for them explicitly (wait_vm_lgkm0).
__device__ __forceinline__ void dma16(unsigned lds_byte_addr, unsigned voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_byte_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

__device__ __forceinline__ unsigned lds_addr(const uint4* p) {
  return (unsigned)reinterpret_cast<unsigned long long>((__attribute__((address_space(3))) const uint4*)p);
}

// s_waitcnt with vmcnt(N), lgkmcnt(0), expcnt unchanged (gfx9 encoding:
// vmcnt[3:0] bits 3:0, expcnt bits 6:4, lgkmcnt bits 11:8, vmcnt[5:4] bits 15:14).
template <int N> __device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier that also keeps the compiler from moving memory accesses
// across it; the caller's explicit waits make the LDS data visible.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// One MFMA operand fragment (8 bf16 or 4 fp32 k values of one tile row, the
// same k assignment as a K-contiguous chunk) from a NAT tile in LDS: `step`
// addresses the step's k rows, off[] holds the lane's byte offsets of its
// reads (nat_lane_byte_bf16 / _f32).
__device__ __forceinline__ uint4 nat_frag(const char* step, const int* off, bf16) {
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const short* src = reinterpret_cast<const short*>(step + off[h]);
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)src);
    w[2 * h] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
    w[2 * h + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ uint4 nat_frag(const char* step, const int* off, float) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = *reinterpret_cast<const uint32_t*>(step + off[e]);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ int nat_lane_byte(int rb, int h, int lane, int rc, bf16) {
  return nat_lane_byte_bf16(rb, h, lane, rc);
}
__device__ __forceinline__ int nat_lane_byte(int rb, int h, int lane, int rc, float) {
  return nat_lane_byte_f32(rb, h, lane, rc);
}

// OCC workgroups of WM x WN waves per CU: at least OCC WM WN / 4 waves on
// each of the CU's four SIMDs (HIP's second launch bound), which caps the
// VGPRs.  Every wave runs MFMAs and issues its share of the K stages' loads.
// NG > 1: the launch covers up to NG groups of slices of different shapes
// (GemmLaunch); the workgroup's group is found from its logical tile id.
template <typename T, int BM, int BN, int WM, int WN, int CPR, int ST, int OCC, int MODE, int PL, int QL, int NG,
          bool LATE>
__global__ __launch_bounds__(WM* WN * 64, (OCC * WM * WN + 3) / 4) void gemm_kernel(
    const GemmLaunch<NG> L) {
  // operand layouts (OperandLayout): which read paths each operand needs
  constexpr bool PNAT = PL == LAY_NAT, QNAT = QL == LAY_NAT;
  constexpr bool P_KC = PL != LAY_NAT, P_NT = PL != LAY_KCONT;  // K-contiguous / natural reads of P
  constexpr bool Q_KC = QL != LAY_NAT, Q_NT = QL != LAY_KCONT;
  constexpr bool HAS_SYM = PL == LAY_SYM || QL == LAY_SYM;
  constexpr int NW = WM * WN, NT = NW * 64;  // every wave of the workgroup
  constexpr int EPC = Elem<T>::kChunk;
  constexpr int ES = (int)sizeof(T);
  constexpr int BK = CPR * EPC;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int SM = WTM / 32, SN = WTN / 32;
  constexpr int LP = BM * CPR, LQ = BN * CPR;  // chunks of each operand per stage
  constexpr int STAGE = LP + LQ;
  constexpr int NIW = STAGE / 64 / NW;         // load instructions per wave per stage
  constexpr int ERC = epi_row_chunks(BN, ES);  // staged output row, in chunks
  constexpr int RCP = BM / EPC, RCQ = BN / EPC;  // chunks per k row of a NAT tile
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(!mode_is_tri(MODE) || BM == BN, "triangle modes need square tiles");
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "4, 8 or 16 chunks per LDS row");
  static_assert(LP % 64 == 0 && STAGE % (64 * NW) == 0, "stage must split into whole wave loads");
  static_assert(ST >= 2 && NIW * (ST - 2) < 64, "ring depth");
  static_assert(!LATE || !mode_is_tri(MODE), "late load issue: update tiles only");

  __shared__ uint4 lds[lds_chunks(BM, BN, CPR, ST, ES)];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;

  int grp = 0, lin;
  if constexpr (NG > 1) lin = xcd_group_tile(blockIdx.x, gridDim.x, L.start, L.n, &grp);
  else lin = xcd_remap(blockIdx.x, gridDim.x);
  const GemmArgs& g = L.g[grp];
  const int slice = lin / g.tiles_per_slice;
  const int q = lin - slice * g.tiles_per_slice;
  int ti, tj;
  if (mode_is_tri(MODE)) tri_decode(q, g.tiles_m, ti, tj);
  else rect_decode(q, g.tiles_m, g.tiles_n, ti, tj);
  const int i0 = ti * BM, j0 = tj * BN;
  // diagonal triangle tiles with 2 x 4 MFMA waves: SIMD-balanced wave
  // columns, and no MFMAs for blocks wholly above the diagonal (tri_wave_col).
  // Not the 256 tile on natural-layout operands (the tall Gram): it already
  // spills, and the skip made it slower.
  constexpr bool DIAG_SKIP = mode_is_tri(MODE) && WM == 2 && WN == 4 && !(BM == 256 && PL == LAY_NAT);
  const int wn = DIAG_SKIP ? tri_wave_col(wm, wave % WN, WN, ti == tj) : wave % WN;
  uint32_t above = 0;  // bit a * SN + b: block (a, b) is not computed
  if (DIAG_SKIP && ti == tj) {
#pragma unroll
    for (int a = 0; a < SM; ++a)
#pragma unroll
      for (int b = 0; b < SN; ++b)
        if (tri_block_above(wm, wn, a, b, SM, SN)) above |= 1u << (a * SN + b);
  }
  // first stage an operand reads in its natural layout (never: a large value)
  const int nat_from_p = PL == LAY_SYM ? sym_nat_from(i0, g.sym_tile, BK) : (PNAT ? 0 : 0x7fffffff);
  const int nat_from_q = QL == LAY_SYM ? sym_nat_from(j0, g.sym_tile, BK) : (QNAT ? 0 : 0x7fffffff);

  // Buffer descriptors over the two operand slices: an offset at or past the
  // slice end reads as zero, which fills rows past M / N and k past K.
  const T* Pbase = reinterpret_cast<const T*>(g.P) + (size_t)slice * g.p_bs;
  const T* Qbase = reinterpret_cast<const T*>(g.Q) + (size_t)slice * g.q_bs;
  const i32x4 rP = make_rsrc(Pbase, (unsigned)(g.p_bs * ES));
  const i32x4 rQ = make_rsrc(Qbase, (unsigned)(g.q_bs * ES));
  constexpr unsigned kOutOfRange = 0x80000000u;

  // Per-lane source of each of this wave's load instructions: the byte
  // offset at k0 = 0 (past the slice end for rows past M / N), K-contiguous
  // or natural per the operand's layout, plus the natural-layout offset of a
  // LAY_SYM operand.  From one stage to the next an operand's offsets move by
  // a wave-uniform step.
  unsigned src_off[NIW], src_alt[HAS_SYM ? NIW : 1];
  auto src_of = [&](const DmaSrc& d, bool nat) __attribute__((always_inline)) -> unsigned {
    const int ld = d.is_p ? g.ldp : g.ldq;
    const int g_row = (d.is_p ? i0 : j0) + d.row;  // tile row (KCONT) or column (NAT)
    const bool ok = g_row < (d.is_p ? g.M : g.N);
    const size_t off = nat ? ((size_t)d.kpos * ld + g_row) * ES : ((size_t)g_row * ld + d.kpos) * ES;
    return ok ? (unsigned)off : kOutOfRange;
  };
#pragma unroll
  for (int t = 0; t < NIW; ++t) {
    const int idx = wave * NIW + t;
    src_off[t] = src_of(dma_src(idx, lane, BM, BN, CPR, EPC, PNAT, QNAT, ES), idx * 64 < LP ? PNAT : QNAT);
    if constexpr (HAS_SYM) src_alt[t] = src_of(dma_src(idx, lane, BM, BN, CPR, EPC, true, true, ES), true);
  }
  // A diagonal Gram or poly tile reads the same rows as P and as Q (the
  // Gram: rows or columns of X; the poly: rows of A): its stages load the P
  // rows only, spread over every wave, and its Q fragments are read from the
  // P region.  With A stored as its lower block triangle both operands switch
  // layouts at the same stage (i0 == j0).  (The 2-slot ring waits for all of
  // a wave's loads at every stage, so a wave's load count may differ between
  // tiles.)
  constexpr bool DSH = (MODE == MODE_GRAM || MODE == MODE_POLY) && ST == 2 && PL == QL;
  constexpr bool DSH_SYM = DSH && PL == LAY_SYM;
  constexpr int NIP = NIW / 2;  // P loads per wave, spread over every wave
  static_assert(!DSH || (BM == BN && NIP * 2 == NIW), "diagonal sharing needs square tiles");
  const bool dshare = DSH && ti == tj;
  unsigned src_dg[DSH ? NIP : 1], src_dga[DSH_SYM ? NIP : 1];
  if constexpr (DSH) {
#pragma unroll
    for (int t = 0; t < NIP; ++t) {
      src_dg[t] = src_of(dma_src(wave * NIP + t, lane, BM, BN, CPR, EPC, PNAT, QNAT, ES), PNAT);
      if constexpr (DSH_SYM) src_dga[t] = src_of(dma_src(wave * NIP + t, lane, BM, BN, CPR, EPC, true, true, ES), true);
    }
  }
  const unsigned step_kc = (unsigned)(BK * ES);
  const unsigned step_np = (unsigned)(BK * g.ldp * ES), step_nq = (unsigned)(BK * g.ldq * ES);
  // Loads of stage kt into ring slot `slot`.  When the whole stage lies
  // inside K (always, for K a multiple of BK) only rows past M / N need the
  // zero fill, and their offset already starts past the slice end; otherwise
  // each lane also checks its own k position.
  // part: -1 every load of the wave, 0 / 1 the first / second half of them
  auto issue = [&](int kt, int slot, auto part) __attribute__((always_inline)) {
    constexpr int PART = decltype(part)::value;
    auto mine = [&](int t) __attribute__((always_inline)) { return PART < 0 || (t < NIW / 2) == (PART == 0); };
    const int k0 = kt * BK;
    // natural-layout reads this stage (compile-time unless LAY_SYM)
    const bool pn = PL == LAY_SYM ? kt >= nat_from_p : PNAT;
    const bool qn = QL == LAY_SYM ? kt >= nat_from_q : QNAT;
    auto off_of = [&](int t, bool is_p) __attribute__((always_inline)) -> unsigned {
      const bool nat = is_p ? pn : qn;
      const bool alt = HAS_SYM && (is_p ? PL == LAY_SYM : QL == LAY_SYM) && nat;
      return (alt ? src_alt[HAS_SYM ? t : 0] : src_off[t]) + (unsigned)kt * (nat ? (is_p ? step_np : step_nq) : step_kc);
    };
    if (DSH && dshare) {
#pragma unroll
      for (int t = 0; t < (DSH ? NIP : 1); ++t) {
        const int idx = wave * NIP + t;  // P chunks only, in this stage's layout (pn == qn here)
        const unsigned base = (DSH_SYM && pn) ? src_dga[DSH_SYM ? t : 0] : src_dg[DSH ? t : 0];
        const unsigned off = base + (unsigned)kt * (pn ? step_np : step_kc);
        const int kpos = dma_src(idx, lane, BM, BN, CPR, EPC, pn, qn, ES).kpos;
        dma16(lds_addr(lds + slot * STAGE + idx * 64), (k0 + BK <= g.K || k0 + kpos < g.K) ? off : kOutOfRange, rP);
      }
    } else if (k0 + BK <= g.K) {
#pragma unroll
      for (int t = 0; t < NIW; ++t) {
        if (!mine(t)) continue;
        const int idx = wave * NIW + t;  // wave-uniform
        const bool is_p = idx * 64 < LP;
        dma16(lds_addr(lds + slot * STAGE + idx * 64), off_of(t, is_p), is_p ? rP : rQ);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NIW; ++t) {
        if (!mine(t)) continue;
        const int idx = wave * NIW + t;
        const bool is_p = idx * 64 < LP;
        const int kpos = dma_src(idx, lane, BM, BN, CPR, EPC, pn, qn, ES).kpos;
        dma16(lds_addr(lds + slot * STAGE + idx * 64), (k0 + kpos < g.K) ? off_of(t, is_p) : kOutOfRange,
              is_p ? rP : rQ);
      }
    }
  };

  f32x16 acc[SM][SN];
#pragma unroll
  for (int a = 0; a < SM; ++a)
#pragma unroll
    for (int b = 0; b < SN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const int l32 = lane & 31;

  // Per-lane byte offsets of the fragment reads; every read of the K loop is
  // one of them plus a compile-time offset (kc_lane_byte, nat_lane_byte_*).
  constexpr int KS = CPR / 2;                      // MFMA k steps per stage
  constexpr int NH = sizeof(T) == 2 ? 2 : 4;       // LDS reads per NAT fragment
  constexpr int QOFF = LP * 16;                    // Q region within a stage
  constexpr int NSP = nat_step_bytes(RCP, ES), NSQ = nat_step_bytes(RCQ, ES);
  static_assert(CPR == 4 || CPR == 8, "fragment addressing assumes 4 or 8 chunks per row");
  int kcp[P_KC ? KS : 1], kcq[Q_KC ? KS : 1];
  int natp[P_NT ? SM : 1][NH], natq[Q_NT ? SN : 1][NH];
  if constexpr (P_KC) {
#pragma unroll
    for (int s = 0; s < KS; ++s) kcp[s] = kc_lane_byte(wm * WTM, s, lane, CPR);
  }
  if constexpr (P_NT) {
#pragma unroll
    for (int a = 0; a < SM; ++a)
#pragma unroll
      for (int h = 0; h < NH; ++h) natp[a][h] = nat_lane_byte(wm * WTM + 32 * a, h, lane, RCP, T());
  }
  if constexpr (Q_KC) {
#pragma unroll
    for (int s = 0; s < KS; ++s) kcq[s] = kc_lane_byte(wn * WTN, s, lane, CPR) + QOFF;
  }
  if constexpr (Q_NT) {
#pragma unroll
    for (int b = 0; b < SN; ++b)
#pragma unroll
      for (int h = 0; h < NH; ++h) natq[b][h] = nat_lane_byte(wn * WTN + 32 * b, h, lane, RCQ, T()) + QOFF;
  }
  if (DSH && dshare) {  // Q fragments from the P region (same rows)
    if constexpr (Q_KC) {
#pragma unroll
      for (int s = 0; s < KS; ++s) kcq[s] -= QOFF;
    }
    if constexpr (Q_NT) {
#pragma unroll
      for (int b = 0; b < SN; ++b)
#pragma unroll
        for (int h = 0; h < NH; ++h) natq[b][h] -= QOFF;
    }
  }
  const char* lb = reinterpret_cast<const char*>(lds);
  // fragments of step s; pn / qn (std::integral_constant) select the natural
  // layout reads for this stage
  auto load_step = [&](int slot, int s, auto pn, auto qn, uint4 (&pf)[SM], uint4 (&qf)[SN])
                       __attribute__((always_inline)) {
    const char* st = lb + slot * STAGE * 16;
#pragma unroll
    for (int a = 0; a < SM; ++a) {
      if constexpr (decltype(pn)::value) pf[a] = nat_frag(st + s * NSP, natp[P_NT ? a : 0], T());
      else pf[a] = *reinterpret_cast<const uint4*>(st + kcp[P_KC ? (s ^ kc_sigma(a, CPR)) : 0] + a * 32 * CPR * 16);
    }
#pragma unroll
    for (int b = 0; b < SN; ++b) {
      if constexpr (decltype(qn)::value) qf[b] = nat_frag(st + s * NSQ, natq[Q_NT ? b : 0], T());
      else qf[b] = *reinterpret_cast<const uint4*>(st + kcq[Q_KC ? (s ^ kc_sigma(b, CPR)) : 0] + b * 32 * CPR * 16);
    }
  };
  // The k step after whose MFMAs a wave issues its share of the next
  // stage's loads (-1: at the stage's barrier).  A wave that issues them is
  // held up while its CU's vector-memory path accepts them (about 500
  // cycles when all 8 waves issue 8 KB each at once), so in the bf16
  // update's launches of more than four rounds, and in the 256 x 256 Gram,
  // the waves of tile row half 1 issue one k step after those of half 0:
  // the two waves of a SIMD then take turns, one issuing loads while the
  // other keeps the matrix core busy.  With fewer than 16 K stages the
  // later half of each stage's loads lands too late, and update launches of
  // up to four rounds issue each wave's loads later (LATE): the first half
  // after k step 0, the second after k step 1.  (The 128 x 128 triangle
  // tiles, two workgroups per CU, lose from it: their lower-triangle poly
  // then spills.)
  constexpr bool STAGGER = (MODE == MODE_UPD_ROW || MODE == MODE_UPD_COL || (mode_is_tri(MODE) && BM == 256)) &&
                           ST == 2 && std::is_same<T, bf16>::value;
  constexpr bool SPLIT = LATE && STAGGER;  // (the fp32 instances never take LATE)
  static_assert(!SPLIT || (KS >= 2 && NIW % 2 == 0), "late issue: two k steps, an even load count");
  const int issue_step = !STAGGER || LATE ? -1 : (wm == 1 && (g.K + BK - 1) / BK >= kStaggerMinStages ? 0 : -1);
  // fragments of step s + 1 are read while the MFMAs of step s run
  // `late` issues the next stage's loads (or half of them) after the MFMAs
  // of k step issue_step (LATE: k steps 0 and 1)
  auto compute = [&](int slot, auto pn, auto qn, auto&& late) __attribute__((always_inline)) {
    uint4 pf[2][SM], qf[2][SN];
    load_step(slot, 0, pn, qn, pf[0], qf[0]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) load_step(slot, s + 1, pn, qn, pf[(s + 1) & 1], qf[(s + 1) & 1]);
      // keep the scheduler from sinking these reads back to their uses
      if (NS_FRAG_BARRIER) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < SM; ++a)
#pragma unroll
        for (int b = 0; b < SN; ++b)
          if (!DIAG_SKIP || !((above >> (a * SN + b)) & 1u)) mfma_chunk(acc[a][b], qf[s & 1][b], pf[s & 1][a], T());
      if (SPLIT && s < 2) {
        __builtin_amdgcn_sched_barrier(0);
        if (s == 0) late(std::integral_constant<int, 0>());
        else late(std::integral_constant<int, 1>());
        __builtin_amdgcn_sched_barrier(0);
      } else if (STAGGER && s == issue_step) {
        __builtin_amdgcn_sched_barrier(0);
        late(std::integral_constant<int, -1>());
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  typedef std::integral_constant<bool, true> Nat;
  typedef std::integral_constant<bool, false> Kc;

  // Epilogue operands captured while they pass through LDS.  The update's
  // diagonal term d_C ⊙ X needs X at the output position, which is the
  // operand stage whose k range covers the tile's rows (wide: Q = columns of
  // X, k = output row) or columns (tall: P = rows of X, k = output column):
  // it is folded into the fp32 accumulators there.  The poly epilogue needs
  // O_A at the output position, the P stage at k = output column: kept in
  // registers until the epilogue.
  typedef typename Quad<T>::Raw QRaw;
  const float* din = g.d_in + (size_t)slice * g.d_bs;
  const __amdgpu_buffer_rsrc_t rD =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(din), (short)0, (int)(g.d_bs * 4), 0x00020000);

  // 1 / (||x||_F + eps) from the slice's partial sums of squares (first
  // step only); every wave of every kernel sums them in the same order, so
  // the Gram and the update agree bitwise
  float inv_norm = 1.0f;
  if (MODE != MODE_POLY && g.d_norm != nullptr) {
    const float* dn = g.d_norm + (size_t)slice * g.norm_n;
    float t = 0.0f;
    for (int i = lane; i < g.norm_n; i += 64) t += dn[i];
    t = wave_sum(t);
    inv_norm = 1.0f / (sqrtf(t) + g.eps);
  }
  const float gram_scale = inv_norm * inv_norm;
  const float cb = g.cb, cc = g.cc;
  float drow[SM];
  constexpr bool POLY_CAP = MODE == MODE_POLY;  // O_A quads kept in registers
  QRaw obuf[POLY_CAP ? SM : 1][POLY_CAP ? SN : 1][4];
  if (MODE == MODE_UPD_ROW) {
#pragma unroll
    for (int a = 0; a < SM; ++a) {
      const int i = i0 + wm * WTM + a * 32 + l32;
      drow[a] = i < g.M ? din[i] : 0.0f;
    }
  }
  if (POLY_CAP) {
#pragma unroll
    for (int a = 0; a < SM; ++a)
#pragma unroll
      for (int b = 0; b < SN; ++b)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) obuf[a][b][rg] = QRaw{};
  }
  auto capture = [&](int slot, int kt) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    const uint4* Ps = lds + slot * STAGE;
    const uint4* Qs = Ps + LP;
    if (MODE == MODE_UPD_ROW) {
#pragma unroll
      for (int a = 0; a < SM; ++a) {
        const int ib = i0 + wm * WTM + a * 32;  // wave-uniform, 32-aligned
        if (ib < k0 || ib >= k0 + BK) continue;
        const int kr = ib - k0 + l32;
#pragma unroll
        for (int b = 0; b < SN; ++b)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int jl = wn * WTN + b * 32 + acc_j(rg, lane);
            const int pos = kr * RCQ + ((jl / EPC) ^ nat_swz(kr, RCQ, ES));
            float x[4];
            Quad<T>::unpack(*reinterpret_cast<const QRaw*>(reinterpret_cast<const T*>(Qs + pos) + jl % EPC), x);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[a][b][4 * rg + e] = fmaf(drow[a], x[e], acc[a][b][4 * rg + e]);
          }
      }
    } else if (MODE == MODE_UPD_COL || MODE == MODE_POLY) {
#pragma unroll
      for (int b = 0; b < SN; ++b) {
        const int jb = j0 + wn * WTN + b * 32;  // wave-uniform, 32-aligned
        if (jb < k0 || jb >= k0 + BK) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int j = jb + acc_j(rg, lane);
          const int kk = j - k0;
          // d_C[j .. j+3] through a buffer load: a per-lane offset, the
          // block's column in a scalar and the register group as an
          // immediate (plain pointer arithmetic here is hoisted out of the
          // K loop as eight 64-bit addresses); past N it reads zeros
          float4 dj = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          if (MODE == MODE_UPD_COL)
            dj = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                rD, (unsigned)(acc_j(rg, lane) * 4), (unsigned)(jb * 4), 0));
#pragma unroll
          for (int a = 0; a < SM; ++a) {
            const int il = wm * WTM + a * 32 + l32;
            const QRaw raw = *reinterpret_cast<const QRaw*>(
                reinterpret_cast<const T*>(Ps + lds_swz(il, kk / EPC, CPR)) + kk % EPC);
            if constexpr (MODE == MODE_POLY) {
              if constexpr (POLY_CAP) obuf[a][b][rg] = raw;
            } else {
              float x[4];
              Quad<T>::unpack(raw, x);
              acc[a][b][4 * rg + 0] = fmaf(dj.x, x[0], acc[a][b][4 * rg + 0]);
              acc[a][b][4 * rg + 1] = fmaf(dj.y, x[1], acc[a][b][4 * rg + 1]);
              acc[a][b][4 * rg + 2] = fmaf(dj.z, x[2], acc[a][b][4 * rg + 2]);
              acc[a][b][4 * rg + 3] = fmaf(dj.w, x[3], acc[a][b][4 * rg + 3]);
            }
          }
        }
      }
    }
  };

  // Ring of ST stages: stage kt lives in slot kt % ST.  Before computing
  // stage kt a wave waits until its own loads of stage kt are done (the
  // loads of the up to ST-2 later stages may stay in flight); the barrier
  // then publishes every wave's part, and also certifies that slot
  // (kt-1) % ST is no longer read, so stage kt+ST-1 can be loaded into it.
  // The loop runs in groups of ST stages (then a tail of fewer) so that every
  // slot index, and with it every LDS address, is a compile-time constant.
  // With LAY_SYM operands it runs in up to three phases of fixed layouts,
  // each starting at a multiple of ST (sym_tile / BK is a multiple of ST).
  const int nk = (g.K + BK - 1) / BK;
  auto stage = [&](int kt, int u, auto pn, auto qn) __attribute__((always_inline)) {  // u == kt % ST
    const int after = nk - 1 - kt;   // stages issued after kt, capped at ST-2
    if (after >= ST - 2) wait_vm_lgkm0<NIW * (ST - 2)>();
    else if (ST > 3 && after == 2) wait_vm_lgkm0<NIW * 2>();
    else if (ST > 2 && after == 1) wait_vm_lgkm0<NIW>();
    else wait_vm_lgkm0<0>();
    ring_barrier();
    // the stage's loads go out here, or after the k step issue_step
    auto late = [&](auto part) __attribute__((always_inline)) {
      if (kt + ST - 1 < nk) issue(kt + ST - 1, (u + ST - 1) % ST, part);
    };
    if (issue_step < 0 && !SPLIT) late(std::integral_constant<int, -1>());
    compute(u, pn, qn, late);
    // the poly's O_A capture happens at the stage covering the tile's own
    // columns, left of its diagonal, where P is K-contiguous
    if constexpr (MODE != MODE_GRAM && !(MODE == MODE_POLY && decltype(pn)::value)) capture(u, kt);
  };
  auto phase = [&](int kt_begin, int kt_end, auto pn, auto qn) __attribute__((always_inline)) {  // kt_begin % ST == 0
    int kt0 = kt_begin;
    for (; kt0 + ST <= kt_end; kt0 += ST) {
#pragma unroll
      for (int u = 0; u < ST; ++u) stage(kt0 + u, u, pn, qn);
    }
#pragma unroll
    for (int u = 0; u < ST - 1; ++u)
      if (kt0 + u < kt_end) stage(kt0 + u, u, pn, qn);
  };
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nk) issue(s, s, std::integral_constant<int, -1>());
  if constexpr (PL == LAY_SYM && QL == LAY_SYM) {
    // both operands symmetric: a lower-triangle tile (j0 <= i0) switches Q
    // to natural-layout reads first
    static_assert(mode_is_tri(MODE), "two symmetric operands need j0 <= i0");
    const int np = nat_from_p < nk ? nat_from_p : nk, nq = nat_from_q < nk ? nat_from_q : nk;
    phase(0, nq, Kc(), Kc());
    phase(nq, np, Kc(), Nat());
    phase(np, nk, Nat(), Nat());
  } else if constexpr (PL == LAY_SYM) {
    const int np = nat_from_p < nk ? nat_from_p : nk;
    phase(0, np, Kc(), std::integral_constant<bool, QNAT>());
    phase(np, nk, Nat(), std::integral_constant<bool, QNAT>());
  } else if constexpr (QL == LAY_SYM) {
    const int nq = nat_from_q < nk ? nat_from_q : nk;
    phase(0, nq, std::integral_constant<bool, PNAT>(), Kc());
    phase(nq, nk, std::integral_constant<bool, PNAT>(), Nat());
  } else {
    phase(0, nk, std::integral_constant<bool, PNAT>(), std::integral_constant<bool, QNAT>());
  }
  wait_vm_lgkm0<0>();
  __syncthreads();

  // ------------------------------------------------------------ epilogue
  // 1. fp32 epilogue in registers, converted values staged in LDS as the
  //    BM x BN tile (rows padded by one chunk);
  // 2. direct store of tile rows; 3. transposed store (mirror / Xᵀ).
  T* O = reinterpret_cast<T*>(g.out) + (size_t)slice * g.o_bs;
  float* dout = g.d_out + (size_t)slice * g.d_bs;
  const bool diag_tile = mode_is_tri(MODE) && ti == tj;
  T* S = reinterpret_cast<T*>(lds);
  constexpr int SROW = ERC * EPC;  // staged row stride in elements

  {
#pragma unroll
    for (int a = 0; a < SM; ++a) {
      const int il = wm * WTM + a * 32 + acc_i(lane);
      const int i = i0 + il;
#pragma unroll
      for (int b = 0; b < SN; ++b)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int jl = wn * WTN + b * 32 + acc_j(rg, lane);
          const int j = j0 + jl;
          if (i >= g.M || j >= g.N) continue;  // N % 8 == 0: j..j+3 all valid
          float v[4] = {acc[a][b][4 * rg], acc[a][b][4 * rg + 1], acc[a][b][4 * rg + 2], acc[a][b][4 * rg + 3]};
          float w[4];
          if (MODE == MODE_GRAM) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[e] = v[e] * gram_scale;
              if (i == j + e) {
                dout[i] = w[e];
                w[e] = 0.0f;
              }
            }
          } else if (MODE == MODE_POLY) {
            float o[4];
            Quad<T>::unpack(obuf[POLY_CAP ? a : 0][POLY_CAP ? b : 0][rg], o);
            const float4 dj = *reinterpret_cast<const float4*>(din + j);
            const float dje[4] = {dj.x, dj.y, dj.z, dj.w};
            const float di = din[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // b O_A + c (O_A O_A + (d_i + d_j) O_A); diagonal: a + b d_i + c ((O_A O_A)_ii + d_i^2)
              w[e] = fmaf(cb, o[e], cc * fmaf(di + dje[e], o[e], v[e]));
              if (i == j + e) {
                dout[i] = fmaf(cc, fmaf(di, di, v[e]), fmaf(cb, di, g.ca));
                w[e] = 0.0f;
              }
            }
          } else {
            // d_C ⊙ X was added to the accumulators in the K loop
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = v[e] * inv_norm;
          }
          *reinterpret_cast<typename Quad<T>::Raw*>(S + il * SROW + jl) = Quad<T>::pack(w);
        }
    }
  }
  __syncthreads();

  // 2. direct store: chunk (il, c) = elements il, [8c/4c .. +EPC) of the tile
  constexpr int CPT = BN / EPC;  // chunks per tile row
  for (int qd = tid; qd < BM * CPT; qd += NT) {
    const int il = qd / CPT, c = qd % CPT;
    const int i = i0 + il, j = j0 + c * EPC;
    if (i >= g.M || j >= g.N) continue;
    uint4 val;
    if (diag_tile && c * EPC + EPC - 1 > il) {
      // upper part of a diagonal tile: take the mirror of the lower part
      T tmp[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int jl = c * EPC + e;
        tmp[e] = (jl <= il) ? S[il * SROW + jl] : S[jl * SROW + il];
      }
      val = *reinterpret_cast<const uint4*>(tmp);
    } else {
      val = *reinterpret_cast<const uint4*>(S + il * SROW + c * EPC);
    }
    *reinterpret_cast<uint4*>(O + (size_t)i * g.ldo + j) = val;
  }

  // 3. transposed store (the mirror)
  if (g.out_t != nullptr && !diag_tile) {
    T* OT = reinterpret_cast<T*>(g.out_t) + (size_t)slice * g.ot_bs;
    if constexpr (ES == 2) {
      // transposing LDS reads; each wave store covers 16 output rows with
      // 64 contiguous bytes each (mirror_lane)
      static_assert(BN % 16 == 0 && BM % 32 == 0 && ((BN / 16) * (BM / 32)) % NW == 0, "mirror units");
      for (int u = wave; u < (BN / 16) * (BM / 32); u += NW) {
        const MirrorLane ml = mirror_lane(u, lane, BN);
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const short* src = reinterpret_cast<const short*>(S + ml.src_row[h] * SROW + ml.src_col);
          const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)src);
          w[2 * h] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
          w[2 * h + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
        }
        const int j = j0 + ml.col, i = i0 + ml.row0;
        if (j < g.N && i < g.M)
          *reinterpret_cast<uint4*>(OT + (size_t)j * g.ldt + i) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
      // fp32: column jl of the tile, rows [EPC r .. +EPC)
      constexpr int RCH = BM / EPC;  // chunks per transposed row
      for (int qd = tid; qd < BN * RCH; qd += NT) {
        const int jl = qd % BN, rc = qd / BN;
        const int j = j0 + jl, i = i0 + rc * EPC;
        if (j >= g.N || i >= g.M) continue;
        T tmp[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) tmp[e] = S[(rc * EPC + e) * SROW + jl];
        *reinterpret_cast<uint4*>(OT + (size_t)j * g.ldt + i) = *reinterpret_cast<const uint4*>(tmp);
      }
    }
  }
}

// --------------------------------------------------------- normalisation

__device__ __forceinline__ float sumsq16(uint4 u, bf16) {
  float s = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = u4get(u, d);
    const float lo = bf16_lo(w), hi = bf16_hi(w);
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
    o[d] = pack_bf16(bf16_lo(w) * inv, bf16_hi(w) * inv);
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
__device__ __forceinline__ void sumsq_block(const NormArgs& g, int slice, int chunk) {
  __shared__ float red[kNormThreads / 64];
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
template <typename T>
__global__ __launch_bounds__(kNormThreads) void sumsq_kernel(const NormArgs g) {
  sumsq_block<T>(g, blockIdx.y, blockIdx.x);
}
// several stacks in one launch (NormLaunch): a 1-D grid of blocks
template <typename T>
__global__ __launch_bounds__(kNormThreads) void sumsq_grouped_kernel(const NormLaunch<kMaxLaunchGroups> L) {
  const int b = blockIdx.x;
  const int grp = launch_group(b, L.start, L.n);
  const NormArgs& g = L.a[grp];
  const int local = b - L.start[grp];
  sumsq_block<T>(g, local / g.chunks, local % g.chunks);
}

// Pass 2: every block sums its slice's partials (same order in every block),
// then writes x / (sqrt(sum) + eps) for the same 32 KiB block, in place if
// y == x (each element is read and written by the same thread).
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

// --------------------------------------------------- padding (odd shapes)

// Bytes [sh, sh + 16) of the 32 bytes lo:hi (sh a multiple of 2, below 16).
__device__ __forceinline__ uint4 bytes_at(uint4 lo, uint4 hi, unsigned sh) {
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  const unsigned q = sh >> 2, b = sh & 3;
  uint32_t win[5];  // dwords q .. q + 4
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const uint32_t a = (q & 1) ? w[k + 1] : w[k];
    const uint32_t c = (q & 1) ? w[k + 3] : w[k + 2];
    win[k] = (q & 2) ? c : a;
  }
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = __builtin_amdgcn_alignbyte(win[k + 1], win[k], b);
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// v with its bytes from nb on (nb a multiple of 2, below 16) set to zero.
__device__ __forceinline__ uint4 keep_bytes(uint4 v, unsigned nb) {
  uint32_t o[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int left = (int)nb - 4 * k;  // bytes of dword k to keep
    o[k] = left >= 4 ? o[k] : left <= 0 ? 0u : (o[k] & 0xffffu);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// The zero-padded copy of a slice and its partial sums of squares in one
// pass.  Block (chunk, slice) covers the same vectors of the padded slice,
// thread by thread, as sumsq_kernel does over the padded copy, so the
// partials are bitwise the ones that kernel would compute from it.  The
// caller's rows are not 16-byte aligned: each vector's elements are taken
// from the one or two aligned 16-byte blocks of the caller's array that hold
// them, read whole and shifted into place, and zeroed past the row's end.
// (The array starts 16-byte aligned, so each such block holds a byte of the
// array; its last block may run up to 14 bytes past the end, in the same
// page.)
template <typename T>
__global__ __launch_bounds__(kNormThreads) void pad_sumsq_kernel(const PadArgs p, const NormArgs g) {
  __shared__ float red[kNormThreads / 64];
  constexpr int EPV = Elem<T>::kChunk, ES = (int)sizeof(T);
  const int slice = blockIdx.y, chunk = blockIdx.x;
  const char* src = reinterpret_cast<const char*>(p.src) + (size_t)slice * p.urows * p.ucols * ES;
  uint4* dst = reinterpret_cast<uint4*>(p.dst) + (size_t)slice * g.slice_vecs;
  const int vpr = (int)(p.cols / EPV), urows = (int)p.urows, ucols = (int)p.ucols;
  const int v0 = (int)((long long)chunk * g.chunk_vecs);
  const int v1 = (int)((v0 + g.chunk_vecs < g.slice_vecs) ? v0 + g.chunk_vecs : g.slice_vecs);
  // the aligned block holding the array's last byte: the second block of a
  // vector is read from no further than here (beyond it, its bytes are unused)
  const uint4* last = reinterpret_cast<const uint4*>(
      (reinterpret_cast<uintptr_t>(p.src) + (size_t)p.batch * p.urows * p.ucols * ES - 1) & ~(uintptr_t)15);
  // four vectors per round: every load of a round is issued before the first
  // is used (the sum still runs over the vectors in order)
  constexpr int U = 4;
  float s = 0.0f;
  for (int vb = v0 + (int)threadIdx.x; vb < v1; vb += U * kNormThreads) {
    uint4 lo[U], hi[U];
    unsigned sh[U], nb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = vb + u * kNormThreads;
      int i, j0;
      pad_vec(v, vpr, EPV, &i, &j0);
      lo[u] = hi[u] = make_uint4(0u, 0u, 0u, 0u);
      sh[u] = 0;
      nb[u] = 0;  // bytes of the caller's row in this vector (0: none)
      if (v < v1 && i < urows && j0 < ucols) {
        const int n = ucols - j0 < EPV ? ucols - j0 : EPV;
        const char* a = src + ((size_t)i * ucols + j0) * ES;
        sh[u] = (unsigned)(reinterpret_cast<uintptr_t>(a) & 15);
        nb[u] = (unsigned)(n * ES);
        const uint4* al = reinterpret_cast<const uint4*>(a - sh[u]);
        lo[u] = al[0];
        hi[u] = al + 1 < last ? al[1] : *last;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = vb + u * kNormThreads;
      if (v >= v1) break;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (nb[u]) {
        val = bytes_at(lo[u], hi[u], sh[u]);
        if (nb[u] < 16) val = keep_bytes(val, nb[u]);
      }
      dst[v] = val;
      s += sumsq16(val, T());
    }
  }
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

// The caller's block out of a padded result.  The caller's array is taken as
// one flat run of 16-byte blocks (it starts 16-byte aligned): one block per
// thread (grid-stride in x over the blocks whose first element lies in slice
// blockIdx.y), stored whole, or element by element where it runs past the
// array's end.  A block whose elements lie in one row of the padded
// slice (rows 16-byte aligned there) takes them from the one or two aligned
// 16-byte blocks of that row that hold them; one that spans two rows gathers
// them element by element.
template <typename T>
__global__ __launch_bounds__(256) void unpad_kernel(const PadArgs p) {
  constexpr int EPV = Elem<T>::kChunk, ES = (int)sizeof(T);
  const long long per_slice = p.urows * p.ucols, total = p.batch * per_slice;
  const int urows = (int)p.urows, ucols = (int)p.ucols;
  const T* src = reinterpret_cast<const T*>(p.src);
  T* dst = reinterpret_cast<T*>(p.dst);
  const long long base = (long long)blockIdx.y * per_slice;           // the slice's first element
  const long long b0 = (base + EPV - 1) / EPV, b1 = (base + per_slice + EPV - 1) / EPV;
  for (long long blk = b0 + (long long)blockIdx.x * 256 + threadIdx.x; blk < b1; blk += (long long)gridDim.x * 256) {
    const long long e0 = blk * EPV;
    long long sl = blockIdx.y;
    const int r = (int)(e0 - base);
    int i = r / ucols, j = r - i * ucols;
    if (j + EPV <= ucols && e0 + EPV <= total) {
      const char* row = reinterpret_cast<const char*>(src + (sl * p.rows + i) * p.cols);
      const unsigned sh = (unsigned)(j * ES) & 15u;
      const uint4* al = reinterpret_cast<const uint4*>(row + (j * ES - (int)sh));
      const uint4 lo = al[0];
      const uint4 hi = sh ? al[1] : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(dst + e0) = bytes_at(lo, hi, sh);
      continue;
    }
    T e[EPV];
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      e[k] = e0 + k < total ? src[(sl * p.rows + i) * p.cols + j] : T(0.0f);
      if (++j == ucols) {
        j = 0;
        if (++i == urows) {
          i = 0;
          ++sl;
        }
      }
    }
    if (e0 + EPV <= total) {
      uint4 val;
      __builtin_memcpy(&val, e, 16);
      *reinterpret_cast<uint4*>(dst + e0) = val;
    } else {
#pragma unroll
      for (int k = 0; k < EPV; ++k)
        if (e0 + k < total) dst[e0 + k] = e[k];
    }
  }
}

// ------------------------------------------------------------- launchers

// Timing events of the launches this thread makes next (set_launch_events).
// They ride in the dispatch itself (hipExtLaunchKernelGGL): the start event
// takes the first dispatch's start, the stop event every dispatch's end (the
// last one stands), and no marker packet goes between the kernels.
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

void set_launch_events(hipEvent_t start, hipEvent_t stop) {
  t_ev_start = start;
  t_ev_stop = stop;
}

template <typename K, typename... A>
static void dispatch(K kernel, dim3 grid, dim3 block, hipStream_t st, A... args) {
  if (t_ev_start == nullptr && t_ev_stop == nullptr) {
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
    return;
  }
  hipExtLaunchKernelGGL(kernel, grid, block, 0, st, t_ev_start, t_ev_stop, 0, args...);
  t_ev_start = nullptr;  // a later launch of the same kind moves only the stop
}

// A launch over the groups gs[0 .. n): one group is a plain launch (NG = 1);
// several go out kMaxLaunchGroups at a time, each launch's grid covering the
// tiles of its groups.
template <typename T, int MODE, int CLS, int PL, int QL, bool LATE = false>
static hipError_t launch_mode(const GemmArgs* gs, int n, hipStream_t st) {
  constexpr TileCfg t = tile_cfg(std::is_same<T, bf16>::value ? 1 : 0, mode_is_tri(MODE), CLS);
  const dim3 block(t.wm * t.wn * 64);
  if (n == 1) {
    GemmLaunch<1> L{};
    L.g[0] = gs[0];
    L.n = 1;
    dispatch(gemm_kernel<T, t.bm, t.bn, t.wm, t.wn, t.cpr, t.st, t.occ, MODE, PL, QL, 1, LATE>,
             dim3(gs[0].tiles_per_slice * gs[0].batch), block, st, L);
    return hipGetLastError();
  }
  static_assert(sizeof(GemmLaunch<kMaxLaunchGroups>) <= 4096, "kernel arguments over 4 KiB");
  for (int g0 = 0; g0 < n;) {
    GemmLaunch<kMaxLaunchGroups> L{};
    long long total = 0;
    const int k = launch_chunk(
        n - g0, [&](int i) { return (long long)gs[g0 + i].tiles_per_slice * gs[g0 + i].batch; }, L.start, &total);
    for (int i = 0; i < k; ++i) L.g[i] = gs[g0 + i];
    L.n = k;
    dispatch(gemm_kernel<T, t.bm, t.bn, t.wm, t.wn, t.cpr, t.st, t.occ, MODE, PL, QL, kMaxLaunchGroups, LATE>,
             dim3((unsigned)total), block, st, L);
    if (hipError_t e = hipGetLastError()) return e;
    g0 += k;
  }
  return hipSuccess;
}

template <typename T, int MODE, int PL, int QL>
static hipError_t launch_tri(int cls, const GemmArgs* gs, int n, hipStream_t st) {
  if (!std::is_same<T, bf16>::value) return launch_mode<T, MODE, TRI_NARROW, PL, QL>(gs, n, st);
  switch (cls) {
    case TRI_WIDE: return launch_mode<T, MODE, TRI_WIDE, PL, QL>(gs, n, st);
    case TRI_BIG: return launch_mode<T, MODE, TRI_BIG, PL, QL>(gs, n, st);
    default: return launch_mode<T, MODE, TRI_NARROW, PL, QL>(gs, n, st);
  }
}

// The late load issue of the update (late_issue): bf16 launches of at most
// kLateIssueMaxTiles tiles over all their groups, or with no group long
// enough for the staggered issue.
template <typename T>
static bool late_issue_of(const GemmArgs* gs, int n) {
  long long tiles = 0;
  int max_k = 0;
  for (int i = 0; i < n; ++i) {
    tiles += (long long)gs[i].tiles_per_slice * gs[i].batch;
    max_k = std::max(max_k, gs[i].K);
  }
  return late_issue(std::is_same<T, bf16>::value ? 1 : 0, tiles, max_k);
}

template <typename T>
static hipError_t dispatch_mode(const StageKind& k, const GemmArgs* gs, int n, hipStream_t st) {
  auto late_issue = [](const GemmArgs* g, int m) { return late_issue_of<T>(g, m); };
  const bool wide = k.tri_cls == TRI_WIDE && std::is_same<T, bf16>::value;
  switch (k.mode) {
    case MODE_GRAM:
      if (k.p_nat) return launch_tri<T, MODE_GRAM, LAY_NAT, LAY_NAT>(k.tri_cls, gs, n, st);
      return launch_tri<T, MODE_GRAM, LAY_KCONT, LAY_KCONT>(k.tri_cls, gs, n, st);
    case MODE_POLY:
      // the poly never takes the big tile (see tri_class)
      // lower-triangle reads of A: bf16, 128 tile (see TileChoice)
      if (k.p_sym && k.q_sym && std::is_same<T, bf16>::value && !wide)
        return launch_mode<bf16, MODE_POLY, TRI_NARROW, LAY_SYM, LAY_SYM>(gs, n, st);
      if (k.p_sym || k.q_sym) return hipErrorInvalidValue;
      return wide ? launch_mode<T, MODE_POLY, TRI_WIDE, LAY_KCONT, LAY_KCONT>(gs, n, st)
                  : launch_mode<T, MODE_POLY, TRI_NARROW, LAY_KCONT, LAY_KCONT>(gs, n, st);
    case MODE_UPD_ROW:
      if (k.p_sym || k.q_sym) return hipErrorInvalidValue;
      return late_issue(gs, n) ? launch_mode<T, MODE_UPD_ROW, TRI_NARROW, LAY_KCONT, LAY_NAT, true>(gs, n, st)
                               : launch_mode<T, MODE_UPD_ROW, TRI_NARROW, LAY_KCONT, LAY_NAT>(gs, n, st);
    case MODE_UPD_COL:
      if (k.p_sym || k.q_sym) return hipErrorInvalidValue;
      return late_issue(gs, n) ? launch_mode<T, MODE_UPD_COL, TRI_NARROW, LAY_KCONT, LAY_KCONT, true>(gs, n, st)
                               : launch_mode<T, MODE_UPD_COL, TRI_NARROW, LAY_KCONT, LAY_KCONT>(gs, n, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int dtype, const StageKind& k, const GemmArgs& g, hipStream_t st) {
  if (dtype == 1) return dispatch_mode<bf16>(k, &g, 1, st);
  return dispatch_mode<float>(k, &g, 1, st);
}

hipError_t launch_gemm_grouped(int dtype, const StageKind& k, const GemmArgs* gs, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (dtype == 1) return dispatch_mode<bf16>(k, gs, n, st);
  return dispatch_mode<float>(k, gs, n, st);
}

hipError_t launch_pad_sumsq(int dtype, const PadArgs& p, const NormArgs& g, int batch, hipStream_t st) {
  dim3 grid(g.chunks, batch);
  if (dtype == 1) dispatch(pad_sumsq_kernel<bf16>, grid, dim3(kNormThreads), st, p, g);
  else dispatch(pad_sumsq_kernel<float>, grid, dim3(kNormThreads), st, p, g);
  return hipGetLastError();
}

hipError_t launch_unpad(int dtype, const PadArgs& p, hipStream_t st) {
  const int epv = elems_per_chunk(dtype);
  const long long blocks = (p.urows * p.ucols + epv - 1) / epv + 1;  // 16-byte blocks starting in one slice
  const long long want = (blocks + 255) / 256;
  const unsigned bx = (unsigned)(want < 65536 ? want : 65536);
  if (dtype == 1) dispatch(unpad_kernel<bf16>, dim3(bx, (unsigned)p.batch), dim3(256), st, p);
  else dispatch(unpad_kernel<float>, dim3(bx, (unsigned)p.batch), dim3(256), st, p);
  return hipGetLastError();
}

hipError_t launch_sumsq(int dtype, const NormArgs& g, int batch, hipStream_t st) {
  dim3 grid(g.chunks, batch);
  if (dtype == 1) dispatch(sumsq_kernel<bf16>, grid, dim3(kNormThreads), st, g);
  else dispatch(sumsq_kernel<float>, grid, dim3(kNormThreads), st, g);
  return hipGetLastError();
}

hipError_t launch_sumsq_grouped(int dtype, const NormArgs* gs, const int* batch, int n, hipStream_t st) {
  if (n == 1) return launch_sumsq(dtype, gs[0], batch[0], st);  // the plain (slice, block) grid
  for (int g0 = 0; g0 < n;) {
    NormLaunch<kMaxLaunchGroups> L{};
    long long total = 0;
    const int k = launch_chunk(
        n - g0, [&](int i) { return (long long)gs[g0 + i].chunks * batch[g0 + i]; }, L.start, &total);
    for (int i = 0; i < k; ++i) L.a[i] = gs[g0 + i];
    L.n = k;
    if (dtype == 1) dispatch(sumsq_grouped_kernel<bf16>, dim3((unsigned)total), dim3(kNormThreads), st, L);
    else dispatch(sumsq_grouped_kernel<float>, dim3((unsigned)total), dim3(kNormThreads), st, L);
    if (hipError_t e = hipGetLastError()) return e;
    g0 += k;
  }
  return hipSuccess;
}

hipError_t launch_scale(int dtype, const NormArgs& g, int batch, hipStream_t st) {
  dim3 grid(g.chunks, batch);
  if (dtype == 1) dispatch(scale_kernel<bf16>, grid, dim3(kNormThreads), st, g);
  else dispatch(scale_kernel<float>, grid, dim3(kNormThreads), st, g);
  return hipGetLastError();
}

}  // namespace ns
