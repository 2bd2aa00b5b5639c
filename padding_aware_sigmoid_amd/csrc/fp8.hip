// FP8 (OCP E4M3) path of padding-aware sigmoid attention: per-tile
// quantisation, and a forward on gfx950's FP8 MFMA.
//
// Method: the sigmoid forward (gist.science summary of arXiv:2604.27124,
// section 2.A; rainbus.top summary, "方法步骤详情", steps 1-3) on quantised
// operands, the FP8 direction the pages leave as future work (rainbus.top
// summary, "未来方向"; paperlayer.ai summary, section 5).
//
// Quantisation (all steps exact but the final rounding):
//  - Q, K and V are quantised per tile of 64 rows of one (sample, head), rows
//    counted from the sample's first row. A tile's scale is the power of two
//    2^E with E = floor(log2 amax) - 7 (amax * 2^-E in [128, 256), so no code
//    overflows), E = 0 for an all-zero tile, E >= -127. It is stored as the
//    byte E + 127 (E8M0), one per (sample, head, tile).
//  - A code is x * 2^-E rounded to nearest-even E4M3 by v_cvt_pk_fp8_f32.
//  - Before P V, P is quantised per query row and per 64-key tile the same
//    way, from the largest P of the tile's valid keys.
//
// CDNA4 design:
//  - Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32
//    accumulation). The E8M0 scale operands carry every power-of-two scale
//    for free: K's and Q's tile scales in S^T = K Q^T, P's row scale and V's
//    tile scale in O = P V.
//  - P's scale 2^e folds into sigma's constants:
//    2^-e sigma(S) = 1 / (2^e + 2^(c1 s + c0 + e)), so the scaled weight costs
//    the same VALU work as the unscaled one.
//  - Workgroups, waves and tiles as the bf16 forward: 4 waves of 64 query rows,
//    64-key K and V tiles by DMA into LDS, two slots each (K two tiles ahead,
//    V one; one __shared__ variable per slot, loop unrolled by two), S of tile
//    t+1 on the MFMAs beside sigma of tile t, then P V of tile t beside the
//    masking and scale of tile t+1.
//  - LDS rows are D bytes of 16-byte chunks, chunk c of row r stored at
//    c ^ f8_swz(r): the row reads of K and the transposed reads of V
//    (ds_read_b64_tr_b8) are free of bank conflicts.
//  - Keys at or past n_k are read as zero rows and masked to -inf before the
//    tile maximum, so their weight is exactly 0 and P's scale comes from valid
//    keys only.
#include <algorithm>

#include "common.hpp"

namespace sigattn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int D>
struct F8Cfg {
  static constexpr int BQ = 256;        // query rows per workgroup (4 waves of 64)
  static constexpr int BK = 64;         // keys per LDS tile
  static constexpr int KS = D / 64;     // MFMA k-steps of 64 over the head dim
  static constexpr int NB = D / 32;     // 32-wide column blocks of O
  static constexpr int CPR = D / 16;    // 16-byte chunks per row
  static constexpr int TILE = BK * D;   // bytes of one K (or V) tile
};
constexpr int kF8Tile = 64;   // rows per quantisation tile
constexpr int kE8M0One = 127; // E8M0 byte of 2^0
// Key tiles per sample whose scale bytes the forward stages in LDS: L <= 262144.
constexpr int kF8MaxTiles = 4096;

// LDS bank groups (16 bytes) of chunk c of row r are spread by an XOR of c
// with f8_swz(r). LDS serves 16 lanes of 16-byte reads (or 32 lanes of 8-byte
// reads) per 256-byte phase. D = 128: rows are 128 bytes, two per phase; the
// K row reads (16 consecutive rows, one chunk) and the transposed V reads
// (rows {0-3, 8-11} + 4h, two adjacent chunks) each hit 16 distinct groups.
// D = 64: rows are 64 bytes, four per phase.
template <int D>
__device__ __forceinline__ int f8_swz(int r) {
  if constexpr (D == 128) {
    const int k = (r >> 1) & 7;
    return ((k & 1) << 2) | (k >> 1);
  } else {
    return (r >> 2) & 3;
  }
}

template <int D>
__device__ __forceinline__ int f8_off(int r, int c) {
  return r * D + ((c ^ f8_swz<D>(r)) << 4);
}

// One 32-byte MFMA operand: chunks c and c + 1 of row r.
template <int D>
__device__ __forceinline__ i32x8 lds8_row(const uint8_t* tile, int r, int c) {
  const i32x4 lo = *(const i32x4*)(tile + f8_off<D>(r, c));
  const i32x4 hi = *(const i32x4*)(tile + f8_off<D>(r, c + 1));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// V^T as the B operand of O = P V for column block db: lane (d = 32 db + l%32,
// half h) byte i holds V[key(h, i)][d], key(h, i) = 32 (i/16) + 8 ((i%16)/4)
// + 4h + i%4, the key order of P's bytes (S^T accumulator registers). Four
// ds_read_b64_tr_b8 give bytes 8t .. 8t + 7. Within a 16-lane group, lane i
// receives byte i%8 of the chunks addressed by lanes 2j + i/8 (j = 0..7,
// measured on the device), so lane m of the group addresses row key(h, 8t + m/2),
// column d0 + 8 (m % 2), d0 = 32 db + 16 ((lane / 16) % 2).
template <int D>
__device__ __forceinline__ i32x8 lds8_vt(const uint8_t* tile, int db, int lane) {
  const int g = lane >> 4, m = lane & 15, h = lane >> 5, j = m >> 1;
  const int col = 32 * db + 16 * (g & 1) + 8 * (m & 1);
  i32x8 out;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 32 * (t >> 1) + 16 * (t & 1) + 8 * (j >> 2) + 4 * h + (j & 3);
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(tile + f8_off<D>(row, col >> 4) + (col & 15)));
    out[2 * t] = v[0];
    out[2 * t + 1] = v[1];
  }
  return out;
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  // format 0 = E4M3 for both operands; sa, sb are E8M0 scale bytes (row of A, column of B)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// DMA 64 rows of D bytes into a swizzled LDS tile; rows at or past n_valid arrive
// as zeros because they lie past the end of the buffer resource. As for the bf16
// tiles, the tile moves in chunks of 256 16-byte slots (RPC whole rows each); a
// lane's offset within its chunk is the same in every chunk (RPC is a multiple
// of the swizzle's 16-row period), and each chunk has its own resource, based
// at its first row and ending at its last valid row.
template <int D>
__device__ __forceinline__ void dma_tile8(uint8_t* tile, const uint8_t* rows, uint32_t row_bytes, int n_valid,
                                          int tid) {
  constexpr int CPR = D / 16, RPC = 256 / CPR;
  static_assert(64 % RPC == 0 && RPC % 16 == 0, "chunks must hold whole swizzle periods and split the tile");
  const int r0 = tid / CPR, c0 = (tid % CPR) ^ f8_swz<D>(r0);
  const uint32_t voff = (uint32_t)r0 * row_bytes + ((uint32_t)c0 << 4);
  const int wbase = __builtin_amdgcn_readfirstlane(tid) & ~63;
#pragma unroll
  for (int i = 0; i < 64 / RPC; ++i) {
    const int nvi = n_valid - i * RPC;
    const int nv = nvi < 0 ? 0 : (nvi > RPC ? RPC : nvi);
    const i32x4 rsrc = make_rsrc(rows + (size_t)(i * RPC) * row_bytes, nv > 0 ? (uint32_t)(nv - 1) * row_bytes + D : 0u);
    llvm_amdgcn_raw_buffer_load_lds(
        rsrc, (lds_u32_ptr)((__attribute__((address_space(3))) char*)tile + (i * 256 + wbase) * 16), 16, (int)voff, 0,
        0, 0);
  }
}

// Largest of 16 accumulator values.
__device__ __forceinline__ float max16(const f32x16& s) {
  float a = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  float b = fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]));
  float c = fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11]));
  float d = fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Power-of-two exponent of a tile with largest magnitude amax: floor(log2 amax) - 7, 0 for 0, >= -127.
__device__ __forceinline__ int tile_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 8;
  return e < -127 ? -127 : e;
}

// ------------------------------------------------------------------------------------- quantiser
// A block of 256 threads per (sample, head, 64-row tile), grid-stride. Each
// thread takes 8-element pieces of the tile's rows: amax by block reduction,
// then the codes. Rows of the tile past n (still inside the tensor) get code 0.
template <int D>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const __bf16* __restrict__ X, uint8_t* __restrict__ X8,
                                                           uint8_t* __restrict__ scales, SeqLayout sl, int Z, int H,
                                                           int use_k) {
  constexpr int PR = D / 8, PIECES = kF8Tile * PR;  // 8-element pieces per row, per tile
  __shared__ float red[4];
  const int ntiles = (sl.L + kF8Tile - 1) / kF8Tile;
  const long long items = (long long)Z * H * ntiles;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (long long item = blockIdx.x; item < items; item += gridDim.x) {
    const int m = (int)(item % ntiles);
    const int h = (int)((item / ntiles) % H);
    const int z = (int)(item / ((long long)ntiles * H));
    const int n = use_k ? sl.nk(z) : sl.nq(z);
    const size_t row0 = use_k ? sl.row0_k(z) : sl.row0_q(z);
    const int rows = sl.rows(n);
    const int r0 = m * kF8Tile;
    const size_t rs = (size_t)H * D;
    const __bf16* xb = X + (row0 * H + h) * D;
    uint8_t* qb = X8 + (row0 * H + h) * D;
    float amax = 0.0f;
    for (int p = tid; p < PIECES; p += 256) {
      const int r = r0 + p / PR;
      if (r < n) {
        const bf16x8 v = *(const bf16x8*)(xb + (size_t)r * rs + (p % PR) * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)v[j]));
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (lane == 0) red[w] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();  // red is reused by the next item
    const int e = tile_exp(amax);
    for (int p = tid; p < PIECES; p += 256) {
      const int r = r0 + p / PR;
      if (r >= rows) continue;
      int2 out = make_int2(0, 0);
      if (r < n) {
        const bf16x8 v = *(const bf16x8*)(xb + (size_t)r * rs + (p % PR) * 8);
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = __builtin_amdgcn_ldexpf((float)v[j], -e);
        out.x = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false), true);
        out.y = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false), true);
      }
      *(int2*)(qb + (size_t)r * rs + (p % PR) * 8) = out;
    }
    if (tid == 0) scales[((size_t)z * H + h) * ntiles + m] = (uint8_t)(e + kE8M0One);
  }
}

// ---------------------------------------------------------------------------------------- forward
template <int D>
__global__ __launch_bounds__(256, kWavesPerSimd<D>) void fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                                      const uint8_t* __restrict__ V, const uint8_t* __restrict__ sQ,
                                                      const uint8_t* __restrict__ sK, const uint8_t* __restrict__ sV,
                                                      __bf16* __restrict__ O, SeqLayout sl, int Z, int H, float c1,
                                                      float c0_base) {
  using C = F8Cfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[C::TILE];
  __shared__ uint8_t sSK[kF8MaxTiles];
  __shared__ uint8_t sSV[kF8MaxTiles];
  __shared__ RankLds rank_lds;
  const int n_qt = (sl.L + C::BQ - 1) / C::BQ;
  const int ntiles = (sl.L + kF8Tile - 1) / kF8Tile;
  const TileCoord tc = schedule_tile(blockIdx.x, Z, H, n_qt, sl, rank_lds);
  const int z = tc.z, h = tc.h, m0 = tc.m;
  const int nq = sl.nq(z), nk = sl.nk(z);
  const float c0 = sl.c0_for(c0_base, nk);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)H * D;  // bytes per row of the FP8 tensors, elements per row of O
  const size_t base = (sl.row0_q(z) * H + h) * D;
  const size_t base_k = (sl.row0_k(z) * H + h) * D;
  const uint8_t* sKz = sK + ((size_t)z * H + h) * ntiles;
  const uint8_t* sVz = sV + ((size_t)z * H + h) * ntiles;
  const int rows = sl.rows(nq);
  __bf16* Ob = O + base;
  const int q0 = m0 * C::BQ;

  if (q0 >= nq) {
    const int rows_here = min(C::BQ, rows - q0);
    const bf16x8 zz = zero_bf16x8();
    for (int c = tid; c < rows_here * (D / 8); c += 256)
      *(bf16x8*)(Ob + (size_t)(q0 + c / (D / 8)) * rs + (c % (D / 8)) * 8) = zz;
    return;
  }

  // Q as the B operand of S^T = K Q^T: query row q0 + 64w + 32qb + l32, bytes 64s + 32 half .. + 31.
  i32x8 qf[2][C::KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = q0 + 64 * w + 32 * qb + l32;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const i32x4* p = (const i32x4*)(Q + base + (size_t)qr * rs + 64 * s + 32 * half);
      const i32x4 lo = qr < nq ? p[0] : i32x4{0, 0, 0, 0};
      const i32x4 hi = qr < nq ? p[1] : i32x4{0, 0, 0, 0};
      qf[qb][s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  const int mq = (q0 + 64 * w) / kF8Tile;  // the wave's Q tile
  const int sq_byte = mq < ntiles ? sQ[((size_t)z * H + h) * ntiles + mq] : kE8M0One;

  f32x16 oacc[2][C::NB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.0f;

  // Exactly the key tiles below n_k are computed, each once: tile 0's scores
  // in the prologue, then one iteration per tile, the last of which computes
  // no next-tile scores.
  const int nkt = (nk + C::BK - 1) / C::BK;
  if (nkt > 0) {
    const uint32_t row_bytes = (uint32_t)rs;
    const uint8_t* Kb = K + base_k;
    const uint8_t* Vb = V + base_k;
    auto fetch = [&](uint8_t* dst, const uint8_t* src, int tile) {
      const int k0 = tile * C::BK;
      const size_t off = (size_t)(k0 < nk ? k0 : 0) * rs;  // no row is read past n_k
      dma_tile8<D>(dst, src + off, row_bytes, nk - k0, tid);
    };
    // Scale bytes of the K and V tiles, staged in LDS once: read per tile from
    // their own LDS arrays they need no wait on the DMA in flight (a vector
    // load per tile would). Tiles at or past n_k take scale 2^0.
    for (int i = tid; i < nkt; i += 256) {
      sSK[i] = sKz[i];
      sSV[i] = sVz[i];
    }
    auto tile_scale = [&](const uint8_t* arr, int t) -> int { return t < nkt ? (int)arr[t] : kE8M0One; };
    // S^T of one tile: sacc[kb][qb] register r = score of key 32kb + acc_row(r, half), query 32qb + l32.
    auto scores = [&](f32x16 (&sacc)[2][2], const uint8_t* kt, int sk_byte) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][0][r] = sacc[kb][1][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          const i32x8 a = lds8_row<D>(kt, 32 * kb + l32, 4 * s + 2 * half);
          sacc[kb][0] = mfma8(a, qf[0][s], sacc[kb][0], sk_byte, sq_byte);
          sacc[kb][1] = mfma8(a, qf[1][s], sacc[kb][1], sk_byte, sq_byte);
        }
      }
    };
    // Tile t sits in slot (t + odd) mod 2, odd = (nkt - 1) mod 2, so that the
    // pairs of the loop below end on the last tile, in slot 0.
    const int nb = nkt - 1;
    const bool odd = nb & 1;
    fetch(odd ? sK1 : sK0, Kb, 0);
    fetch(odd ? sV1 : sV0, Vb, 0);
    if (nkt > 1) fetch(odd ? sK0 : sK1, Kb, 1);
    dma_wait();
    __syncthreads();
    f32x16 s_a[2][2], s_b[2][2];
    // P's scale per query row of a tile: from the largest score of its 64 keys
    // (this lane's 32 and the other half's); alpha > 0, so sigma is increasing
    // in s. Keys at or past n_k are masked to -inf first.
    float c0e[2], pe[2];
    int pbyte[2];
    auto mask_and_scale = [&](f32x16 (&sc)[2][2], int key0) {
      if (key0 + C::BK > nk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = key0 + 32 * kb + acc_row(r, half) < nk;
            sc[kb][0][r] = ok ? sc[kb][0][r] : -__builtin_inff();
            sc[kb][1][r] = ok ? sc[kb][1][r] : -__builtin_inff();
          }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = fmaxf(max16(sc[0][qb]), max16(sc[1][qb]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float pmax = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(mx, c1, c0)));
        const int e = tile_exp(pmax);
        c0e[qb] = c0 + (float)e;
        pe[qb] = __builtin_amdgcn_ldexpf(1.0f, e);
        pbyte[qb] = e + kE8M0One;
      }
    };

    // One tile, as a fixed step schedule (one wave per SIMD hides latency only
    // inside its own instruction stream):
    //   S phase:  S(t+1) = K(t+1) Q^T, 4 KS MFMAs || P(t) = 2^-e sigma(S(t)), 64
    //             weights per lane, packed as E4M3 in lds8_vt's key order
    //   PV phase: O += P(t) V(t), 2 NB MFMAs     || mask and scale of S(t+1)
    // Two slots each for K and V: K runs two tiles ahead (tile t+2 goes into
    // tile t's K slot, last read by S(t) in the previous iteration), V one tile
    // ahead (tile t+1 into tile t-1's V slot). Slot X = t % 2 holds K(t) and
    // V(t); Y = 1 - X holds K(t+1) and V(t-1). The last tile's iteration
    // (NEXT false) has no tile t+1: no DMA, no S MFMAs, only P and P V. The
    // DMA of a tile past n_k fills its slot with zeros, which nothing reads.
    constexpr int NS = 4 * C::KS, NP = 2 * C::NB;
    auto iteration = [&](auto next_c, uint8_t* kx, uint8_t* ky, uint8_t* vx, uint8_t* vy, int t,
                         f32x16 (&sc)[2][2], f32x16 (&sn)[2][2]) __attribute__((always_inline)) {
      constexpr bool NEXT = decltype(next_c)::value;
      dma_wait();       // this wave's DMAs of K(t+1) and V(t) have landed
      __syncthreads();  // ... everyone's have, and every wave is done with K(t) and V(t-1)
      if constexpr (NEXT) {
        fetch(kx, Kb, t + 2);
        fetch(vy, Vb, t + 1);
      }
      const int skb = tile_scale(sSK, t + 1), svb = tile_scale(sSV, t);
      const uint8_t* kt = ky;
      const uint8_t* vt = vx;
      i32x8 p8[2];
      float pw[4];
      // Every LDS operand of the tile is requested up front: K(t+1) for the S
      // phase and V(t)^T for the P V phase, so no MFMA waits on a read.
      i32x8 a_ops[2][C::KS], b_ops[C::NB];
      if constexpr (NEXT) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s = 0; s < C::KS; ++s) a_ops[kb][s] = lds8_row<D>(kt, 32 * kb + l32, 4 * s + 2 * half);
      }
#pragma unroll
      for (int db = 0; db < C::NB; ++db) b_ops[db] = lds8_vt<D>(vt, db, lane);
      static_for<0, NS>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int kb = g / (2 * C::KS), s = (g / 2) % C::KS, qb = g % 2;
        if constexpr (!NEXT) {
        } else if constexpr (s == 0) {
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.0f;
          sn[kb][qb] = mfma8(a_ops[kb][s], qf[qb][s], z, skb, sq_byte);
        } else {
          sn[kb][qb] = mfma8(a_ops[kb][s], qf[qb][s], sn[kb][qb], skb, sq_byte);
        }
        constexpr int e0 = g * 64 / NS, e1 = (g + 1) * 64 / NS;
        static_for<e0, e1>([&](auto ec) {
          constexpr int e = decltype(ec)::value;
          constexpr int eq = e / 32, j = (e % 32) / 4, u = e % 4, ekb = j >> 2, er = 4 * (j & 3) + u;
          pw[u] = __builtin_amdgcn_rcpf(pe[eq] + __builtin_amdgcn_exp2f(__builtin_fmaf(sc[ekb][eq][er], c1, c0e[eq])));
          if constexpr (u == 3)
            p8[eq][j] = __builtin_amdgcn_cvt_pk_fp8_f32(pw[2], pw[3],
                                                        __builtin_amdgcn_cvt_pk_fp8_f32(pw[0], pw[1], 0, false), true);
        });
        sched_step<g, 0, NEXT ? 1 : 0, (e1 - e0) * 9 / 2, kNoFence>();
      });
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, NP>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int db = g / 2, qb = g % 2;
        oacc[qb][db] = mfma8(p8[qb], b_ops[db], oacc[qb][db], pbyte[qb], svb);
        sched_step<g, 0, 1, 8, kNoFence>();
      });
      if constexpr (NEXT) mask_and_scale(sn, (t + 1) * C::BK);
    };
    using NX = std::true_type;
    using LAST = std::false_type;
    // Tile 0's scores; with an odd count tile 0 also runs its iteration here
    // (slot 1) and leaves tile 1's scores in s_a. Then tiles in whole pairs up
    // to nkt - 2, then the last tile (slot 0). A loop entered in the middle of
    // a pair, or leftover iterations after it, made the compiler spill or
    // shuffle registers in the loop.
    int t = 0;
    if (odd) {
      scores(s_b, sK1, tile_scale(sSK, 0));
      mask_and_scale(s_b, 0);
      iteration(NX{}, sK1, sK0, sV1, sV0, 0, s_b, s_a);
      t = 1;
    } else {
      scores(s_a, sK0, tile_scale(sSK, 0));
      mask_and_scale(s_a, 0);
    }
    for (; t < nb; t += 2) {
      iteration(NX{}, sK0, sK1, sV0, sV1, t, s_a, s_b);
      iteration(NX{}, sK1, sK0, sV1, sV0, t + 1, s_b, s_a);
    }
    iteration(LAST{}, sK0, sK1, sV0, sV1, nb, s_a, s_b);
    dma_wait();  // the last DMAs (all zeros) must not outlive the kernel
  }

  // Register r of oacc[qb][db] holds query row 64w + 32qb + acc_row(r, half), column 32db + l%32.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = q0 + 64 * w + 32 * qb + acc_row(r, half);
        if (row < rows) Ob[(size_t)row * rs + db * 32 + l32] = (__bf16)(row < nq ? oacc[qb][db][r] : 0.0f);
      }
}

// ---------------------------------------------------------------------------------------- launchers
template <int D>
hipError_t launch_quantize_fp8(const void* x, void* x8, uint8_t* scales, SeqLayout sl, int Z, int H, int use_k,
                               hipStream_t st) {
  const long long items = (long long)Z * H * ((sl.L + kF8Tile - 1) / kF8Tile);
  const unsigned blocks = (unsigned)std::min<long long>(items, 1 << 16);
  hipLaunchKernelGGL(quantize_fp8_kernel<D>, dim3(blocks), dim3(256), 0, st, (const __bf16*)x, (uint8_t*)x8, scales,
                     sl, Z, H, use_k);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8, const uint8_t* sq, const uint8_t* sk,
                          const uint8_t* sv, void* o, SeqLayout sl, int Z, int H, float c1, float c0,
                          hipStream_t st) {
  using C = F8Cfg<D>;
  const long long blocks = (long long)Z * H * ((sl.L + C::BQ - 1) / C::BQ);
  hipLaunchKernelGGL(fwd_fp8_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st, (const uint8_t*)q8,
                     (const uint8_t*)k8, (const uint8_t*)v8, sq, sk, sv, (__bf16*)o, sl, Z, H, c1, c0);
  return hipGetLastError();
}

#define SIGATTN_INST_FP8(D)                                                                                      \
  template hipError_t launch_quantize_fp8<D>(const void*, void*, uint8_t*, SeqLayout, int, int, int, hipStream_t); \
  template hipError_t launch_fwd_fp8<D>(const void*, const void*, const void*, const uint8_t*, const uint8_t*,    \
                                        const uint8_t*, void*, SeqLayout, int, int, float, float, hipStream_t);
SIGATTN_INST_FP8(64)
SIGATTN_INST_FP8(128)

}  // namespace sigattn
