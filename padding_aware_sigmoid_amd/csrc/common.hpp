// Device helpers shared by the sigmoid-attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sigattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// 32x32x16 bf16 MFMA, fp32 accumulate (v_mfma_f32_32x32x16_bf16).
// Lane l of a wave64 supplies:
//   A: row l%32, k = 8*(l/32) + 0..7;
//   B: column l%32, k = 8*(l/32) + 0..7.
// Accumulator register r of lane l holds row (r/4)*8 + 4*(l/32) + r%4 and
// column l%32. These layouts were checked on the device against a host product.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The row an accumulator register maps to (see mfma32).
__device__ __forceinline__ constexpr int acc_row(int r, int half) { return (r >> 2) * 8 + 4 * half + (r & 3); }

// Key (or query) order inside one 16-wide k-step when an accumulator is
// reused as an A operand. k-slot 8*half + j of the operand holds
// accumulator register 8*ks + j, i.e. row 16*ks + 8*(j/4) + 4*half + j%4.
// The B operand fed with it must therefore use the same row order. The
// transposed LDS read below does exactly that.

// sigma(alpha * s + bias) for a raw dot product s, as 1 / (1 + 2^(c1*s + c0))
// with c1 = -alpha*log2(e) and c0 = -bias*log2(e). It uses v_exp_f32 (2^x) and
// v_rcp_f32. If 2^(...) overflows to +inf the result is exactly 0. If it
// underflows to 0 the result is exactly 1. No NaN can arise from finite s.
__device__ __forceinline__ float sigmoid_dot(float s, float c1, float c0) {
  const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(s, c1, c0));
  return __builtin_amdgcn_rcpf(1.0f + t);
}

// sigma with one transcendental, for scores far below 0. With t = e^S =
// 2^(-c1*s - c0), sigma(S) = t / (1 + t) = t - t^2 + t^3 / (1 + t), so t - t^2
// (one FMA) is short by t^3 / (1 + t), a relative error of exactly t^2: at
// most 2^-10, a quarter of P's bf16 rounding step, while t <= 2^-5
// (S <= -3.47). The bias b = -ln n of
// the method puts nearly every score there (S ~ b + N(0, 1) for unit-variance
// inputs, b = -9 at n = 8192). The caller keeps the bit pattern of the
// largest t in tmax (t >= 0, so unsigned order is float order, and a NaN t
// compares above the bound) and recomputes with sigmoid_dot every weight of
// a block in which some lane's tmax exceeds kSmallSigmaMaxBits.
constexpr uint32_t kSmallSigmaMaxBits = 0x3D000000u;  // bits of 2^-5

__device__ __forceinline__ float sigmoid_dot_small(float s, float c1, float c0, uint32_t& tmax) {
  const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(s, -c1, -c0));
  tmax = max(tmax, __float_as_uint(t));
  return __builtin_fmaf(-t, t, t);
}

// One of the two, chosen at compile time.
template <bool SMALL>
__device__ __forceinline__ float sigmoid_pass(float s, float c1, float c0, uint32_t& tmax) {
  if constexpr (SMALL) return sigmoid_dot_small(s, c1, c0, tmax);
  else return sigmoid_dot(s, c1, c0);
}

// Whether some lane of the wave saw a t above the bound (a wave-uniform value).
__device__ __forceinline__ bool small_sigma_out_of_range(uint32_t tmax) {
  return __builtin_amdgcn_ballot_w64(tmax > kSmallSigmaMaxBits) != 0;
}

// A launch with one bias may use sigmoid_dot_small when c0 = -b log2(e) is
// at least this: then a score of 0 (as a zero-filled padded key row gets) has
// t = 2^-c0 <= 2^-6, inside the range, and typical scores are far inside it.
// Below it nearly every block would need the recomputation. With a
// per-sample bias b_z = bias - ln n_k[z] the launch may always use it: the
// kernel's own test on each workgroup's first block of scores (which a
// sample whose zero-filled keys score above the range fails) picks the exact
// form where it does not pay. Neither choice depends on L, so results do not
// change with the amount of padding.
constexpr float kSmallSigmaMinC0 = 6.0f;

__host__ __device__ inline bool use_small_sigma(float c0, int bias_per_sample) {
  return bias_per_sample || c0 >= kSmallSigmaMinC0;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

// Scheduling hint for one region of the key loop: N groups of one MFMA
// followed by up to V VALU instructions. The MFMA pipe then runs beside the
// sigma work instead of in separate bursts. (Mask bits: 0x008 MFMA,
// 0x002 VALU.)
template <int N, int V>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}

// Slot I of a ring of three LDS buffers, chosen at compile time. Each slot is
// its own __shared__ variable. An access through the returned pointer is then
// known to touch only that variable, which lets the compiler tell a DMA into
// one slot apart from reads of another (it waits for an LDS DMA before any LDS
// read it cannot prove disjoint from it).
template <int I, typename T>
__device__ __forceinline__ T* ring(T* a, T* b, T* c) {
  static_assert(I >= 0 && I < 3, "ring slot out of range");
  if constexpr (I == 0) return a;
  else if constexpr (I == 1) return b;
  else return c;
}

// Waves per SIMD a bf16 attention kernel is built for (the second argument of
// __launch_bounds__: the compiler keeps each wave within 512 / that many
// registers). At D = 64 the forward, the fused dK/dV and dQ fit 256 registers
// with a few spills and 49 KB of LDS, so two workgroups share a CU and each
// SIMD interleaves two waves: measured 10-21% faster per kernel on
// cellbatch8k and stress8k than one wave per SIMD without spills. At D = 128
// they need 430-480 registers and 97 KB of LDS: one wave per SIMD.
template <int D>
constexpr int kWavesPerSimd = D == 64 ? 2 : 1;

// Compile-time loop: f(std::integral_constant<int, I>) for I = BEGIN .. END-1.
// The index is a constant expression inside f, which the scheduling builtins
// need.
template <int I, int END, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < END) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, END>(f);
  }
}

// One step of a software-pipelined schedule: NDS LDS reads, NMFMA MFMAs,
// NVALU VALU instructions, in that order. Zero counts are skipped. After
// every FENCE-th step a hard scheduling fence stops later instructions from
// moving up and earlier ones from sinking. Without it the scheduler pairs
// each MFMA with the LDS read right before it, and the read-ahead is lost.
// The VALU work is split evenly behind each MFMA. An MFMA issued right after
// another stalls the in-order wave until the matrix pipe frees, and the VALU
// work placed between them fills those cycles.
constexpr int kNoFence = 1 << 20;  // FENCE value that never fences

template <int J, int NDS, int NMFMA, int NVALU, int FENCE = 2, bool SPLIT = true>
__device__ __forceinline__ void sched_step() {
  if constexpr (NDS > 0) __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
  if constexpr (!SPLIT) {
    if constexpr (NMFMA > 0) __builtin_amdgcn_sched_group_barrier(0x008, NMFMA, 0);
    if constexpr (NVALU > 0) __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);
  } else static_for<0, NMFMA>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    constexpr int v = (m + 1) * NVALU / NMFMA - m * NVALU / NMFMA;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x002, v, 0);
  });
  if constexpr (NMFMA == 0 && NVALU > 0) __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);
  if constexpr (J % FENCE == FENCE - 1) __builtin_amdgcn_sched_barrier(0);
}

// Only the fence of a step: the compiler orders the instructions between two
// fences itself.
template <int J, int FENCE>
__device__ __forceinline__ void sched_fence() {
  if constexpr (J % FENCE == FENCE - 1) __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ int clamp_len(int n, int L) { return n < 0 ? 0 : (n > L ? L : n); }

// Where each sample's rows live, how many are valid, and the score bias.
//  - Padded layout: tensors are [Z, L, H, D]; q and k are the lengths n_q[Z],
//    n_k[Z]. Sample z owns rows z*L .. z*L + L - 1, and rows at or past its
//    length are padding (outputs there are written 0).
//  - Packed layout: tensors are [T, H, D]; q and k are cumulative offsets
//    cu[Z+1]. Sample z owns rows cu[z] .. cu[z+1] - 1, all valid. L bounds
//    every length (longer samples are cut at L).
// Lengths are clamped to [0, L]. With bias_per_sample the bias of sample z is
// bias - ln(n_k[z]) (paperlayer.ai summary, section 3: b = -log n), which
// shifts c0 = -b log2(e) by log2(n_k[z]).
struct SeqLayout {
  const int32_t* q;
  const int32_t* k;
  int L;
  int packed;
  int bias_per_sample;
  __device__ __forceinline__ int len(const int32_t* a, int z) const {
    return clamp_len(packed ? a[z + 1] - a[z] : a[z], L);
  }
  __device__ __forceinline__ int nq(int z) const { return len(q, z); }
  __device__ __forceinline__ int nk(int z) const { return len(k, z); }
  // first row of sample z in Q, O, dO, dQ (row0_q) or in K, V, dK, dV (row0_k)
  __device__ __forceinline__ size_t row0_q(int z) const { return packed ? (size_t)q[z] : (size_t)z * L; }
  __device__ __forceinline__ size_t row0_k(int z) const { return packed ? (size_t)k[z] : (size_t)z * L; }
  // rows of sample z present in the tensors, given its clamped length n
  __device__ __forceinline__ int rows(int n) const { return packed ? n : L; }
  // The result is uniform; readfirstlane keeps it in a scalar register, as the
  // constant c0 is, instead of taking a vector register from the kernel.
  __device__ __forceinline__ float c0_for(float c0, int nk) const {
    const float c = bias_per_sample ? c0 + __builtin_amdgcn_logf((float)(nk > 1 ? nk : 1)) : c0;
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, c)));
  }
};

// ---------------------------------------------------------------------------
// Tile scheduler. A grid covers every (sample z, head h, tile m). Blocks
// whose tile lies wholly in padding exit at once, so the real work per
// (z, h) is proportional to n_q[z] * n_k[z], which can vary widely across a
// padded batch. The mapping block -> (z, h, m):
//  - ranks samples by n_q * n_k, heaviest first (ties by index);
//  - numbers the (sample, head) pairs in that order;
//  - deals the pairs round-robin over the 8 XCDs (block b runs on XCD b % 8).
// Each XCD then gets a similar share of heavy and light pairs and starts with
// its heaviest (longest-processing-time first). All tiles of one pair stay on
// one XCD, so that head's K/V (or Q/dO) stream through one L2; a block-major
// order, which spreads them over the XCDs, measured 20-28% slower on padded
// batches.
// With more than kMaxRankedSamples samples the samples keep their index
// order; when the pair count is not a multiple of 8 the XCD dealing is
// dropped. Every thread of the block calls this (blocks of 256 threads, one
// per sample when ranking), and it contains two barriers. Each thread t < Z
// reads its own sample's lengths once and leaves the weight in LDS; the
// ranks then come from LDS. (Read from global memory inside the ranking
// loop, each of the 2 Z length reads waited for the one before: microseconds
// per workgroup at a few dozen samples, paid by every workgroup, the wholly
// padded ones included.)
constexpr int kMaxRankedSamples = 256;

struct RankLds {
  long long weight[kMaxRankedSamples];  // n_q * n_k of sample t
  int order[kMaxRankedSamples];         // order[rank] = sample
};

struct TileCoord {
  int z, h, m;
};

__device__ __forceinline__ TileCoord schedule_tile(int b, int Z, int H, int ntiles, const SeqLayout& sl,
                                                   RankLds& rank_lds) {
  const int P = Z * H;
  int p, m;
  if ((P & 7) == 0) {
    const int x = b & 7, i = b >> 3;
    p = x + 8 * (i / ntiles);
    m = i % ntiles;
  } else {
    p = b / ntiles;
    m = b % ntiles;
  }
  const int r = p / H, h = p - r * H;
  int z = r;
  if (Z <= kMaxRankedSamples) {
    const int t = threadIdx.x;
    long long wt = 0;
    if (t < Z) {
      wt = (long long)sl.nq(t) * sl.nk(t);
      rank_lds.weight[t] = wt;
    }
    __syncthreads();
    if (t < Z) {
      int rank = 0;
      for (int u = 0; u < Z; ++u) {
        const long long wu = rank_lds.weight[u];
        rank += (wu > wt) || (wu == wt && u < t);
      }
      rank_lds.order[rank] = t;
    }
    __syncthreads();
    z = rank_lds.order[r];
  }
  return {z, h, m};
}

// Keeps the computation of p in the current scheduling region. Without it the
// optimiser sinks register-only arithmetic past the next barrier, towards its
// first use, and the phase loses the VALU work meant to overlap its MFMAs. The
// asm is empty: no instruction, no memory access.
__device__ __forceinline__ void pin_before_barrier(bf16x8 (&p)[2][2]) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) asm volatile("" : "+v"(p[a][b]));
}

// ---------------------------------------------------------------------------
// LDS tiles: 64 rows of D bf16, unpadded. The tile is stored as D / 32 column
// blocks, one after the other; a block holds the 32 columns of every row as
// 64-byte row pieces (four 16-byte chunks), and within a piece the physical
// chunk is the logical one XOR swz(row) = (row >> 2) & 3. Both operand reads
// are conflict-free (16-byte bank groups, 256 bytes per LDS phase):
//  - a natural read (16 lanes, 16 consecutive rows, one chunk each) covers
//    every (row % 4, physical chunk) pair once;
//  - a transposed read (ds_read_b64_tr_b16: 32 lanes, 4 consecutive rows of
//    one block, starting at a multiple of 4) reads 256 contiguous bytes.
// The layout is chosen so that operands at another column block, or 16 rows
// further down, lie at a constant byte distance from the same lane's address:
// only two lane patterns exist per read kind (chunk bit 1 clear or set for
// natural reads, row bit 3 clear or set for transposed reads), and every other
// operand address is one of them plus an immediate offset.
// Whole tiles still arrive by DMA: one column block is 256 16-byte slots, the
// 1 KB per wave instruction of a 256-thread workgroup landing contiguously.
template <int D>
struct Tile {
  static constexpr int ROWS = 64;
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  static constexpr int BLOCK_BYTES = ROWS * 64;
  __device__ static __forceinline__ int swz(int r) { return (r >> 2) & 3; }
  // byte offset of logical chunk c of row r
  __device__ static __forceinline__ int off(int r, int c) {
    return (c >> 2) * BLOCK_BYTES + ((r * 4 + ((c & 3) ^ swz(r))) << 4);
  }
};

// Natural operand: 8 consecutive values of row r starting at logical chunk c.
template <int D>
__device__ __forceinline__ bf16x8 lds_nat(const __bf16* tile, int r, int c) {
  return *(const bf16x8*)((const char*)tile + Tile<D>::off(r, c));
}

// Transposed read feeding the B operand of mfma32 from a tile T[row][col]
// whose rows are the contraction index.
//
// ds_read_b64_tr_b16 works per group of 16 lanes (measured on gfx950). Lane i
// of a group receives, for j = 0..3, element i%4 of the 8-byte chunk that lane
// 4j + i/4 of the same group addresses.
//
// The result: lane l receives T[row0 + 8*part + 4*(l/32) + j][col0 + l%32] for
// j = 0..3, where part 0 and part 1 are the two reads. That is the k-step row
// order described at mfma32.
template <int D>
__device__ __forceinline__ bf16x8 lds_tr(const __bf16* tile, int row0, int col0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = row0 + 4 * (g >> 1) + (s >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  const char* b = (const char*)tile;
  const char* p0 = b + Tile<D>::off(row, col >> 3) + ((col & 7) << 1);
  const char* p1 = b + Tile<D>::off(row + 8, col >> 3) + ((col & 7) << 1);
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// ---------------------------------------------------------------------------
// Global -> LDS DMA (buffer_load_dwordx4 ... lds). Each lane fetches 16 bytes
// at its byte offset into the buffer. The wave's 64 results land contiguously
// at the LDS address of the instruction (lane l at +16*l). A lane whose offset
// lies outside the buffer's range writes zeros (checked on the device).
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned int* lds_u32_ptr;
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(i32x4 rsrc, lds_u32_ptr lds, int size, int voffset,
                                                           int soffset, int offset,
                                                           int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Buffer resource over `bytes` bytes at p (raw, no stride), made wave-uniform.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  i32x4 v;
  v[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  v[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  v[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  v[3] = 0x00020000;  // dword format, as for every gfx9 raw buffer
  return v;
}

constexpr uint32_t kOutOfRange = 0x80000000u;

// DMA a tile's ROWS = 64 rows into LDS. The tile's row i starts at byte
// i * row_bytes after `rows` (row 0 of the tile in global memory). Rows at or
// past n_valid are never read: their lanes lie past the end of the buffer
// resource, which ends at the last valid row, so the LDS receives zeros.
// Every wave of the workgroup takes part. Call dma_wait() before the barrier
// that publishes the tile.
//
// Chunk i moves column block i: thread t fetches row t / 4, physical chunk
// t % 4 of that block (1 KB contiguous in LDS per wave). A thread's offset
// within the block, dma_lane_offset(), is the same for every block; the
// block's 64-byte column shift goes into the chunk's buffer resource (base
// moved by 64 * i bytes, range shortened by as much), so only scalar work and
// no per-lane arithmetic is left per tile. (The instruction's immediate
// offset cannot carry the shift: the DMA adds it to the LDS address too.)
template <int D, int NTHREADS>
__device__ __forceinline__ uint32_t dma_lane_offset(uint32_t row_bytes, int tid) {
  static_assert(NTHREADS == 4 * Tile<D>::ROWS, "one wave instruction per thread moves one column block");
  const int r = tid >> 2, c = (tid & 3) ^ Tile<D>::swz(r);
  return (uint32_t)r * row_bytes + ((uint32_t)c << 4);
}

// One of a tile's D / 32 DMA instructions per thread, chunk i (column block
// i), so that a tile's DMA can be spread over a step schedule instead of
// issued in one burst. Calling every i in 0 .. kDmaChunks - 1 equals dma_tile.
template <int D, int ROWS, int NTHREADS>
constexpr int kDmaChunks = D / 32;

template <int D, int ROWS, int NTHREADS>
__device__ __forceinline__ void dma_tile_chunk(__bf16* tile, const __bf16* rows, uint32_t row_bytes, int n_valid,
                                               int tid, int i) {
  static_assert(ROWS == Tile<D>::ROWS, "tiles are 64 rows");
  const int nv = n_valid < 0 ? 0 : (n_valid > ROWS ? ROWS : n_valid);
  // Valid rows end at byte (nv - 1) * row_bytes + 2 * D of the tile; block i
  // starts at byte 64 * i of each row (64 * i < 2 * D).
  const i32x4 rsrc =
      make_rsrc((const char*)rows + 64 * i, nv > 0 ? (uint32_t)(nv - 1) * row_bytes + 2 * D - 64 * i : 0u);
  const int wbase = __builtin_amdgcn_readfirstlane(tid) & ~63;  // wave-uniform first slot of the chunk
  llvm_amdgcn_raw_buffer_load_lds(
      rsrc, (lds_u32_ptr)((__attribute__((address_space(3))) char*)tile + i * Tile<D>::BLOCK_BYTES + wbase * 16), 16,
      (int)dma_lane_offset<D, NTHREADS>(row_bytes, tid), 0, 0, 0);
}

template <int D, int ROWS, int NTHREADS>
__device__ __forceinline__ void dma_tile(__bf16* tile, const __bf16* rows, uint32_t row_bytes, int n_valid, int tid) {
#pragma unroll
  for (int i = 0; i < kDmaChunks<D, ROWS, NTHREADS>; ++i)
    dma_tile_chunk<D, ROWS, NTHREADS>(tile, rows, row_bytes, n_valid, tid, i);
}

// DMA 64 rows of a float2 row statistic into LDS as float2[64] (512 B). Row r
// of the source sits at byte r * stride_bytes; rows at or past n_valid arrive
// as zeros. Waves 0 and 1 each issue one 4-byte-per-lane instruction (floats
// 0..63, then 64..127); other waves issue nothing.
__device__ __forceinline__ void dma_stats64(float2* dst, const float2* src, uint32_t stride_bytes, int n_valid,
                                            int tid) {
  const int w = tid >> 6, lane = tid & 63;
  if (w >= 2) return;
  const int nv = n_valid < 0 ? 0 : (n_valid > 64 ? 64 : n_valid);
  const i32x4 rsrc = make_rsrc(src, nv > 0 ? (uint32_t)(nv - 1) * stride_bytes + 8 : 0u);
  const int f = w * 64 + lane, row = f >> 1;
  const uint32_t voff = row < nv ? (uint32_t)row * stride_bytes + (uint32_t)(f & 1) * 4 : kOutOfRange;
  llvm_amdgcn_raw_buffer_load_lds(rsrc, (lds_u32_ptr)((__attribute__((address_space(3))) char*)dst + w * 256), 4,
                                  (int)voff, 0, 0, 0);
}

// The same LDS address, with no link to the array it points into that the
// compiler can follow. A DMA into such an address does not make the compiler
// wait for it before reads of that array; the kernel orders the two itself
// (dma_wait, then a barrier, before any read of the DMA's destination). The
// address is workgroup-uniform.
template <typename T>
__device__ __forceinline__ T* lds_opaque(T* p) {
  typedef __attribute__((address_space(3))) char* lds_char_ptr;
  uint32_t a = (uint32_t)(size_t)(lds_char_ptr)p;
  asm volatile("" : "+s"(a));
  return (T*)(lds_char_ptr)(size_t)a;
}

// Wait until this wave's outstanding global loads (the DMAs included) are done.
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

}  // namespace sigattn
