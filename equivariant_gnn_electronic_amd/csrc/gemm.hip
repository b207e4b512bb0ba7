// MFMA GEMMs for the per-|m| SO(2) channel mixing.
//
// The eSCN reduction turns the SO(3) tensor product into linear maps per
// order m (MALOQ Sec. II-B1, Sec. III: "constrained linear layers"); over all
// edges of a layer those maps are dense products with M = number of edges,
// which is the one step of the layer that is a real contraction.
//
// fp32: v_mfma_f32_32x32x2_f32.  Block tile 128x128, 4 waves in a 2x2
// arrangement, 64x64 per wave (2x2 MFMA tiles), K step 16, operands staged
// k-major in LDS (double-buffered) so every fragment read is a
// conflict-free row of LDS.  Tiles are assigned XCD-aware: consecutive
// tiles that share an A row-block are given to workgroups that land on the
// same XCD, so the A block is fetched from HBM once and then hits that
// XCD's L2.
#include "gemm.h"

#include <type_traits>

namespace egnn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 16;
constexpr int PAD = 4;  // LDS row padding (floats)
constexpr int kXcd = 8;

struct TileMap {
  int mt, nt, z;
  bool valid;
};

// Workgroup b runs on XCD b % 8.  Without split-K, XCD x gets the contiguous
// tile range [x*per, (x+1)*per) in (m-major, n-minor) order, so the n-tiles of
// one m-tile share that XCD's L2.  With split-K, every tile of split z runs on
// XCD z % 8: the tiles of one split read the same K-range of both operands,
// which then comes from HBM once instead of once per tile.
__device__ inline TileMap map_tile(int b, int tiles_m, int tiles_n, int splits) {
  const int total = tiles_m * tiles_n;
  const int x = b % kXcd, i = b / kXcd;
  TileMap r;
  int t;
  if (splits == 1) {
    const int per = (total + kXcd - 1) / kXcd;
    t = x * per + i;
    r.z = 0;
    r.valid = t < total;
  } else {
    t = i % total;
    r.z = x + kXcd * (i / total);
    r.valid = r.z < splits;
  }
  r.mt = r.valid ? t / tiles_n : 0;
  r.nt = r.valid ? t % tiles_n : 0;
  return r;
}

// Grid size matching map_tile.
inline int tile_grid(int tiles, int splits) {
  if (splits == 1) return (tiles + kXcd - 1) / kXcd * kXcd;
  return (splits + kXcd - 1) / kXcd * kXcd * tiles;
}

// Operand tiles of ROWS x KT floats move through registers as float4s, NF per
// thread of the 256-thread block (the last one guarded when the tile holds
// fewer than 256 float4s).  In LDS they are laid out [KT][ROWS + PAD].
template <int ROWS, int KT>
struct TileShape {
  static constexpr int F4 = ROWS * KT / 4;            // float4s in the tile
  static constexpr int NF = (F4 + 255) / 256;         // per thread
  static constexpr int LD = ROWS + PAD;               // LDS row length
};

template <bool KCONTIG, int ROWS, int KT>
__device__ inline f32x4 load_f4(const float *P, int ld, int rows, int row0, int k0, int k_end, int f) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (f >= TileShape<ROWS, KT>::F4) return v;
  if (KCONTIG) {
    const int m = f / (KT / 4), kq = f % (KT / 4);
    const int gm = row0 + m, gk = k0 + kq * 4;
    if (gm < rows && gk < k_end) v = *reinterpret_cast<const f32x4 *>(P + static_cast<int64_t>(gm) * ld + gk);
  } else {
    const int k = f / (ROWS / 4), mq = f % (ROWS / 4);
    const int gk = k0 + k, gm = row0 + mq * 4;
    if (gk < k_end && gm < rows) {
      const float *p = P + static_cast<int64_t>(gk) * ld + gm;
      if (gm + 3 < rows) {
        v = *reinterpret_cast<const f32x4 *>(p);
      } else {
        for (int j = 0; j < 4; ++j) v[j] = (gm + j < rows) ? p[j] : 0.f;
      }
    }
  }
  return v;
}

template <bool KCONTIG, int ROWS, int KT>
__device__ inline void store_f4(float *S, const f32x4 &v, int f) {
  using TS = TileShape<ROWS, KT>;
  if (f >= TS::F4) return;
  if (KCONTIG) {
    const int m = f / (KT / 4), kq = f % (KT / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) S[(kq * 4 + j) * TS::LD + m] = v[j];
  } else {
    const int k = f / (ROWS / 4), mq = f % (ROWS / 4);
    *reinterpret_cast<f32x4 *>(S + k * TS::LD + mq * 4) = v;
  }
}

// Block tile (64 TMt) x (64 TNt), 4 waves in a 2 x 2 arrangement, each
// (32 TMt) x (32 TNt) in TMt x TNt MFMA tiles.  The 64-wide variants serve
// dimensions such as 192 and 320 that 128-wide tiles would pad by 25-33%.
template <bool AK, bool BK_, int TMt, int TNt>
__global__ void __launch_bounds__(256, 2) gemm_f32_kernel(int M, int N, int K, const float *__restrict__ A, int lda,
                                                          const float *__restrict__ B, int ldb, float *__restrict__ C,
                                                          int ldc, int splits, int k_per_split, int64_t split_stride) {
  constexpr int TBM = 64 * TMt, TBN = 64 * TNt;
  using SA = TileShape<TBM, BK>;
  using SB = TileShape<TBN, BK>;
  __shared__ float As[2][BK * SA::LD];
  __shared__ float Bs[2][BK * SB::LD];
  const int tiles_m = (M + TBM - 1) / TBM, tiles_n = (N + TBN - 1) / TBN;
  const TileMap tm = map_tile(blockIdx.x, tiles_m, tiles_n, splits);
  if (!tm.valid) return;
  const int z = tm.z;
  const int k_begin = z * k_per_split;
  const int k_end = min(K, k_begin + k_per_split);
  C += z * split_stride;
  const int row0 = tm.mt * TBM, col0 = tm.nt * TBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 32 * TMt, wn = (wave & 1) * 32 * TNt;
  const int fr = lane & 31, fk = lane >> 5;

  f32x16 acc[TMt][TNt];
#pragma unroll
  for (int i = 0; i < TMt; ++i)
#pragma unroll
    for (int j = 0; j < TNt; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  f32x4 ra[SA::NF], rb[SB::NF];
  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < SA::NF; ++h) ra[h] = load_f4<AK, TBM, BK>(A, lda, M, row0, k0, k_end, threadIdx.x + 256 * h);
#pragma unroll
    for (int h = 0; h < SB::NF; ++h) rb[h] = load_f4<BK_, TBN, BK>(B, ldb, N, col0, k0, k_end, threadIdx.x + 256 * h);
  };
  auto store = [&](int b) {
#pragma unroll
    for (int h = 0; h < SA::NF; ++h) store_f4<AK, TBM, BK>(As[b], ra[h], threadIdx.x + 256 * h);
#pragma unroll
    for (int h = 0; h < SB::NF; ++h) store_f4<BK_, TBN, BK>(Bs[b], rb[h], threadIdx.x + 256 * h);
  };
  int buf = 0;
  if (k_begin < k_end) {
    load(k_begin);
    store(0);
  }
  __syncthreads();
  for (int k0 = k_begin; k0 < k_end; k0 += BK) {
    const bool more = k0 + BK < k_end;
    if (more) load(k0 + BK);
    const float *as = As[buf];
    const float *bs = Bs[buf];
    // the fragments of k pair kk + 2 are read from LDS before the products of kk are issued
    float fa[2][TMt], fb[2][TNt];
    auto frag = [&](int kk, float(&a)[TMt], float(&b)[TNt]) {
#pragma unroll
      for (int i = 0; i < TMt; ++i) a[i] = as[(kk + fk) * SA::LD + wm + 32 * i + fr];
#pragma unroll
      for (int j = 0; j < TNt; ++j) b[j] = bs[(kk + fk) * SB::LD + wn + 32 * j + fr];
    };
    frag(0, fa[0], fb[0]);
    // the products issue ahead of the other workgroup's loads and LDS stores
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int st = 0; st < BK / 2; ++st) {
      const int cur = st & 1;
      if (st + 1 < BK / 2) frag(2 * (st + 1), fa[cur ^ 1], fb[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < TMt; ++i)
#pragma unroll
        for (int j = 0; j < TNt; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  // 32x32 accumulator layout: column = lane % 32, row = 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int i = 0; i < TMt; ++i)
#pragma unroll
    for (int j = 0; j < TNt; ++j) {
      const int col = col0 + wn + 32 * j + fr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm + 32 * i + 8 * (r >> 2) + 4 * fk + (r & 3);
        if (row < M) C[static_cast<int64_t>(row) * ldc + col] = acc[i][j][r];
      }
    }
}

// ------------------------------------------------------------------------
// Complex products by Gauss's three-multiplication form.
//
// For |m| >= 1 the SO(2) map is a complex multiplication (W_m1 + i W_m2) by
// (X+ + i X-); its input gradient is a multiplication by the conjugate and
// its weight gradient a sum of conj-products.  All three are
//   Re + i Im = sum_k (U+ + i U-)(m,k) (V+ + i V-)(n,k),
// computed with three real products instead of four:
//   k1 = sum (U+ + U-) V+,  k2 = sum U+ (V- - V+),  k3 = sum U- (V+ + V-),
//   Re = k1 - k3,  Im = k1 + k2.
// U is data with its two halves at a pointer offset; V is either three
// precomputed matrices (V+, V- - V+, V+ + V-) or data whose second half,
// times vsign, is V-.  The sums are formed while a tile goes from registers
// to LDS.  Tile 128 x 128 (per part), K step 8, 4 waves of 64 x 64 x 3 parts.
constexpr int CBK = 8;

template <bool UK, bool VK, bool VPRE, int TMt, int TNt>
__global__ void __launch_bounds__(256, 2) cgemm_f32_kernel(int M, int N, int K, const float *__restrict__ Up,
                                                           const float *__restrict__ Um, int ldu,
                                                           const float *__restrict__ V1, const float *__restrict__ V2,
                                                           const float *__restrict__ V3, int ldv, float vsign,
                                                           float *__restrict__ Cre, float *__restrict__ Cim, int ldc,
                                                           int splits, int k_per_split, int64_t split_stride) {
  constexpr int TBM = 64 * TMt, TBN = 64 * TNt;
  using SU = TileShape<TBM, CBK>;
  using SV = TileShape<TBN, CBK>;
  __shared__ float Us[2][3][CBK * SU::LD];
  __shared__ float Vs[2][3][CBK * SV::LD];
  const int tiles_m = (M + TBM - 1) / TBM, tiles_n = (N + TBN - 1) / TBN;
  const TileMap tm = map_tile(blockIdx.x, tiles_m, tiles_n, splits);
  if (!tm.valid) return;
  const int z = tm.z;
  const int k_begin = z * k_per_split;
  const int k_end = min(K, k_begin + k_per_split);
  Cre += z * split_stride;
  Cim += z * split_stride;
  const int row0 = tm.mt * TBM, col0 = tm.nt * TBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 32 * TMt, wn = (wave & 1) * 32 * TNt;
  const int fr = lane & 31, fk = lane >> 5;

  f32x16 acc[3][TMt][TNt];
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int i = 0; i < TMt; ++i)
#pragma unroll
      for (int j = 0; j < TNt; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][i][j][r] = 0.f;

  f32x4 up[SU::NF], um[SU::NF], va[SV::NF], vb[SV::NF], vc[SV::NF];
  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < SU::NF; ++h) {
      const int f = threadIdx.x + 256 * h;
      up[h] = load_f4<UK, TBM, CBK>(Up, ldu, M, row0, k0, k_end, f);
      um[h] = load_f4<UK, TBM, CBK>(Um, ldu, M, row0, k0, k_end, f);
    }
#pragma unroll
    for (int h = 0; h < SV::NF; ++h) {
      const int f = threadIdx.x + 256 * h;
      va[h] = load_f4<VK, TBN, CBK>(V1, ldv, N, col0, k0, k_end, f);
      vb[h] = load_f4<VK, TBN, CBK>(V2, ldv, N, col0, k0, k_end, f);
      if (VPRE) vc[h] = load_f4<VK, TBN, CBK>(V3, ldv, N, col0, k0, k_end, f);
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int h = 0; h < SU::NF; ++h) {
      const int f = threadIdx.x + 256 * h;
      store_f4<UK, TBM, CBK>(Us[b][0], up[h] + um[h], f);
      store_f4<UK, TBM, CBK>(Us[b][1], up[h], f);
      store_f4<UK, TBM, CBK>(Us[b][2], um[h], f);
    }
#pragma unroll
    for (int h = 0; h < SV::NF; ++h) {
      const int f = threadIdx.x + 256 * h;
      if (VPRE) {
        store_f4<VK, TBN, CBK>(Vs[b][0], va[h], f);
        store_f4<VK, TBN, CBK>(Vs[b][1], vb[h], f);
        store_f4<VK, TBN, CBK>(Vs[b][2], vc[h], f);
      } else {
        const f32x4 vm = vb[h] * vsign;  // V- from the second half
        store_f4<VK, TBN, CBK>(Vs[b][0], va[h], f);
        store_f4<VK, TBN, CBK>(Vs[b][1], vm - va[h], f);
        store_f4<VK, TBN, CBK>(Vs[b][2], va[h] + vm, f);
      }
    }
  };
  int buf = 0;
  if (k_begin < k_end) {
    load(k_begin);
    store(0);
  }
  __syncthreads();
  for (int k0 = k_begin; k0 < k_end; k0 += CBK) {
    const bool more = k0 + CBK < k_end;
    if (more) load(k0 + CBK);
    // steps (k pair, part) in order; the fragments of step s + 1 are read
    // from LDS before the products of step s are issued
    constexpr int NS = (CBK / 2) * 3;
    auto frag = [&](int st, float(&a)[TMt], float(&b)[TNt]) {
      const int kk = 2 * (st / 3), q = st % 3;
      const float *us = Us[buf][q];
      const float *vs = Vs[buf][q];
#pragma unroll
      for (int i = 0; i < TMt; ++i) a[i] = us[(kk + fk) * SU::LD + wm + 32 * i + fr];
#pragma unroll
      for (int j = 0; j < TNt; ++j) b[j] = vs[(kk + fk) * SV::LD + wn + 32 * j + fr];
    };
    float fa[2][TMt], fb[2][TNt];
    frag(0, fa[0], fb[0]);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int cur = st & 1, q = st % 3;
      if (st + 1 < NS) frag(st + 1, fa[cur ^ 1], fb[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < TMt; ++i)
#pragma unroll
        for (int j = 0; j < TNt; ++j)
          acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[cur][i], fb[cur][j], acc[q][i][j], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < TMt; ++i)
#pragma unroll
    for (int j = 0; j < TNt; ++j) {
      const int col = col0 + wn + 32 * j + fr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm + 32 * i + 8 * (r >> 2) + 4 * fk + (r & 3);
        if (row < M) {
          const int64_t o = static_cast<int64_t>(row) * ldc + col;
          Cre[o] = acc[0][i][j][r] - acc[2][i][j][r];
          Cim[o] = acc[0][i][j][r] + acc[1][i][j][r];
        }
      }
    }
}

// ------------------------------------------------------------------------
// bf16 operands, fp32 accumulate: v_mfma_f32_32x32x16_bf16.  Both operands
// K-contiguous; tiles are staged in LDS in the same [row][k] order (rows
// padded by 8 bf16), and each lane reads its 8 consecutive k values of a
// fragment row as one 16-byte LDS read.  Tile 128 x 128, K step 32, 4 waves
// of 64 x 64, XCD-aware tile order as above.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int HBM_ = 128, HBN = 128, HBK = 32, HPAD = 8;
constexpr int HLD = HBK + HPAD;  // LDS row length (bf16)

__device__ inline uint4 load_bf16_chunk(const uint16_t *P, int ld, int rows, int row, int k, int K) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < rows && k < K) v = *reinterpret_cast<const uint4 *>(P + static_cast<int64_t>(row) * ld + k);
  return v;
}

template <bool CBF16>
__global__ void __launch_bounds__(256, 2) gemm_bf16_kernel(int M, int N, int K, const uint16_t *__restrict__ A, int lda,
                                                           const uint16_t *__restrict__ B, int ldb, void *__restrict__ C,
                                                           int ldc) {
  __shared__ uint16_t As[2][HBM_ * HLD];
  __shared__ uint16_t Bs[2][HBN * HLD];
  const int tiles_m = (M + HBM_ - 1) / HBM_, tiles_n = (N + HBN - 1) / HBN;
  const TileMap tm = map_tile(blockIdx.x, tiles_m, tiles_n, 1);
  if (!tm.valid) return;
  const int row0 = tm.mt * HBM_, col0 = tm.nt * HBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  // each thread moves two 16-byte chunks of each 128 x 32 tile: chunk c -> row c / 4, k (c % 4) * 8
  const int c0 = threadIdx.x, c1 = threadIdx.x + 256;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  uint4 ra0, ra1, rb0, rb1;
  auto load = [&](int k0) {
    ra0 = load_bf16_chunk(A, lda, M, row0 + c0 / 4, k0 + (c0 % 4) * 8, K);
    ra1 = load_bf16_chunk(A, lda, M, row0 + c1 / 4, k0 + (c1 % 4) * 8, K);
    rb0 = load_bf16_chunk(B, ldb, N, col0 + c0 / 4, k0 + (c0 % 4) * 8, K);
    rb1 = load_bf16_chunk(B, ldb, N, col0 + c1 / 4, k0 + (c1 % 4) * 8, K);
  };
  auto store = [&](int b) {
    *reinterpret_cast<uint4 *>(&As[b][(c0 / 4) * HLD + (c0 % 4) * 8]) = ra0;
    *reinterpret_cast<uint4 *>(&As[b][(c1 / 4) * HLD + (c1 % 4) * 8]) = ra1;
    *reinterpret_cast<uint4 *>(&Bs[b][(c0 / 4) * HLD + (c0 % 4) * 8]) = rb0;
    *reinterpret_cast<uint4 *>(&Bs[b][(c1 / 4) * HLD + (c1 % 4) * 8]) = rb1;
  };
  int buf = 0;
  if (K > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += HBK) {
    const bool more = k0 + HBK < K;
    if (more) load(k0 + HBK);
#pragma unroll
    for (int kk = 0; kk < HBK; kk += 16) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(&As[buf][(wm + 32 * i + fr) * HLD + kk + fk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[buf][(wn + 32 * j + fr) * HLD + kk + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = col0 + wn + 32 * j + fr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= M) continue;
        const int64_t o = static_cast<int64_t>(row) * ldc + col;
        if (CBF16)
          static_cast<uint16_t *>(C)[o] = f32_to_bf16(acc[i][j][r]);
        else
          static_cast<float *>(C)[o] = acc[i][j][r];
      }
    }
}

// bf16, large tiles, operands brought into LDS by the gfx950 direct loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS
// base + 16 * lane, with no register staging).  S stages form a ring: the
// stage of K-tile i - 1 is refilled with tile i + S - 1 before tile i is
// multiplied, so S - 1 K-tiles are in flight during each product.  Every
// stage (its A tile, then its B tile) is its own LDS object, which lets the
// compiler's wait-count pass see that reads of one stage do not depend on
// the loads still filling the others.  A wave's 1 KB of each load covers
// whole rows of the tile, so rows cannot be padded; instead the 16-byte
// chunks of a row are XOR-swizzled by the row index, which makes the 32-row
// fragment reads conflict-free.
// Requires K % BK == 0, lda and ldb multiples of 8, 16-byte aligned bases.
template <int I, int N, typename F>
__device__ inline void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// vmcnt(n), other counters left alone
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// vmcnt(n) and lgkmcnt(0), before a ring barrier: this wave's direct loads of
// the next K-tile have landed, and its LDS reads of the current stage are
// complete, since other waves start refilling that stage once past the barrier.
template <int N>
__device__ inline void wait_ring() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without the release fence of __syncthreads (the fence
// would wait for every outstanding direct load).  Each wave waits for its
// own loads with wait_vmcnt before arriving; the empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ inline void barrier_no_fence() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <int CPR>
__device__ inline int chunk_swizzle(int row) {
  static_assert(CPR == 4 || CPR == 8, "32 or 64 bf16 per row");
  return CPR == 4 ? ((row >> 2) & 3) : ((row >> 1) & 7);
}

// STAGED (bf16 output only): the MFMA operands are swapped so that a lane
// holds four consecutive output columns of one row; after the main loop each
// wave packs its tile to bf16 in its own slice of the (then idle) ring, rows
// of 128 bytes with XOR-swizzled 16-byte chunks, and writes it back as
// 16-byte stores that cover whole 128-byte lines.  Requires WTN = 64,
// N % 8 == 0, ldc % 8 == 0 and a 16-byte aligned C.  Otherwise each lane
// stores its accumulators one element at a time.
template <int BM, int BN, int BK, int WM, int WN, int S, int U, bool CBF16, bool STAGED>
__global__ void __launch_bounds__(64 * WM * WN, 1) gemm_bf16_lds_kernel(int M, int N, int K,
                                                                      const uint16_t *__restrict__ A, int lda,
                                                                      const uint16_t *__restrict__ B, int ldb,
                                                                      void *__restrict__ C, int ldc, int splits,
                                                                      int k_per_split, int64_t split_stride) {
  constexpr int NW = WM * WN, CPR = BK / 8, ST = (BM + BN) * BK;
  static_assert(S >= 2 && S <= 4, "stages");
  static_assert(!STAGED || CBF16, "staged epilogue writes bf16");
  __shared__ uint16_t T0[ST], T1[ST], T2[S > 2 ? ST : 8], T3[S > 3 ? ST : 8];
  // The wait-count pass has been seen to leave the first direct LDS load it
  // meets in program order without a per-object record, after which every
  // read of that load's stage waits for all loads in flight.  This load never
  // runs (K > 0); it only takes that first place.
  __shared__ __attribute__((aligned(1024))) uint32_t dma_anchor[256];
  if (K < 0) __builtin_amdgcn_global_load_lds(static_cast<const void *>(A), static_cast<void *>(dma_anchor), 16, 0, 0);
  auto ts = [&](auto st) -> uint16_t * {
    if constexpr (decltype(st)::value == 0) return T0;
    else if constexpr (decltype(st)::value == 1) return T1;
    else if constexpr (decltype(st)::value == 2) return T2;
    else return T3;
  };
  auto as = [&](auto st) -> uint16_t * { return ts(st); };
  auto bs = [&](auto st) -> uint16_t * { return ts(st) + BM * BK; };
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const TileMap tm = map_tile(blockIdx.x, tiles_m, tiles_n, splits);
  if (!tm.valid) return;
  // split-K: this block's K range; its partial product goes to slice z of C
  const int k_begin = tm.z * k_per_split;
  const int k_len = max(0, min(K, k_begin + k_per_split) - k_begin);
  C = static_cast<char *>(C) + tm.z * split_stride * (CBF16 ? 2 : 4);
  const int row0 = tm.mt * BM, col0 = tm.nt * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  const int wm = (wave / WN) * WTM, wn = (wave % WN) * WTN;
  const int fr = lane & 31, fh = lane >> 5;
  // direct loads: the A tile is BM * CPR chunks = BM * CPR / 64 wave loads, spread over the waves
  constexpr int LA = BM * CPR / 64 / NW, LB = BN * CPR / 64 / NW;
  static_assert(LA >= 1 && LB >= 1 && (BM * CPR) % (64 * NW) == 0 && (BN * CPR) % (64 * NW) == 0, "tile");
  const uint16_t *ga[LA];
  const uint16_t *gb[LB];
  int la[LA], lb[LB];
#pragma unroll
  for (int h = 0; h < LA; ++h) {
    const int slot0 = (h * NW + wave) * 64, sl = slot0 + lane, r = sl / CPR;
    ga[h] = A + static_cast<int64_t>(min(row0 + r, M - 1)) * lda + k_begin + ((sl % CPR) ^ chunk_swizzle<CPR>(r)) * 8;
    la[h] = slot0 * 8;
  }
#pragma unroll
  for (int h = 0; h < LB; ++h) {
    const int slot0 = (h * NW + wave) * 64, sl = slot0 + lane, r = sl / CPR;
    gb[h] = B + static_cast<int64_t>(min(col0 + r, N - 1)) * ldb + k_begin + ((sl % CPR) ^ chunk_swizzle<CPR>(r)) * 8;
    lb[h] = slot0 * 8;
  }
  auto issue = [&](auto st, int kt) {
#pragma unroll
    for (int h = 0; h < LA; ++h)
      __builtin_amdgcn_global_load_lds(static_cast<const void *>(ga[h] + static_cast<int64_t>(kt) * BK),
                                       static_cast<void *>(as(st) + la[h]), 16, 0, 0);
#pragma unroll
    for (int h = 0; h < LB; ++h)
      __builtin_amdgcn_global_load_lds(static_cast<const void *>(gb[h] + static_cast<int64_t>(kt) * BK),
                                       static_cast<void *>(bs(st) + lb[h]), 16, 0, 0);
  };
  // direct load h of a K-tile (A loads first, then B)
  auto issue_one = [&](auto st, int kt, auto hc) {
    constexpr int h = decltype(hc)::value;
    if constexpr (h < LA)
      __builtin_amdgcn_global_load_lds(static_cast<const void *>(ga[h] + static_cast<int64_t>(kt) * BK),
                                       static_cast<void *>(as(st) + la[h]), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(static_cast<const void *>(gb[h - LA] + static_cast<int64_t>(kt) * BK),
                                       static_cast<void *>(bs(st) + lb[h - LA]), 16, 0, 0);
  };
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto load_frag = [&](auto st, int s, bf16x8(&a)[TM], bf16x8(&b)[TN]) {
    const int c = s * 2 + fh;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm + 32 * i + fr;
      a[i] = *reinterpret_cast<const bf16x8 *>(as(st) + r * BK + (c ^ chunk_swizzle<CPR>(r)) * 8);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn + 32 * j + fr;
      b[j] = *reinterpret_cast<const bf16x8 *>(bs(st) + r * BK + (c ^ chunk_swizzle<CPR>(r)) * 8);
    }
  };
  // hook(q) runs before the q-th MFMA of the K-tile (q = s * TM * TN + i * TN + j)
  auto mma = [&](bf16x8(&a)[TM], bf16x8(&b)[TN], auto sc, auto &&hook) {
    static_for<0, TM * TN>([&](auto qc) {
      constexpr int i = decltype(qc)::value / TN, j = decltype(qc)::value % TN;
      hook(std::integral_constant<int, decltype(sc)::value * TM * TN + decltype(qc)::value>{});
      if constexpr (STAGED)  // output tile transposed: lane = row, registers = columns
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    });
  };
  // one K-tile: the fragments of 16-wide k-step s + 1 are read while step s multiplies
  auto compute = [&](auto st, auto &&hook) {
    bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
    load_frag(st, 0, a0, b0);
    static_for<0, BK / 16>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s % 2 == 0) {
        if constexpr (s + 1 < BK / 16) load_frag(st, s + 1, a1, b1);
        mma(a0, b0, sc, hook);
      } else {
        if constexpr (s + 1 < BK / 16) load_frag(st, s + 1, a0, b0);
        mma(a1, b1, sc, hook);
      }
    });
  };
  constexpr int L = LA + LB;  // direct loads per K-tile per wave
  // The next K-tile's loads go out one at a time between the MFMAs of the first
  // half of the current one: issued as one burst at the top of the tile they
  // held the waves at the memory pipeline while the matrix cores idled.  Load
  // h goes before MFMA slot(h).
  constexpr int NMF = TM * TN * (BK / 16);
  auto slot = [](int h) { return h * (NMF / 2) / L; };
  const int nk = k_len / BK;
  // prologue: K-tiles 0 .. S-2 in flight, wait for tile 0
  static_for<0, S - 1>([&](auto st) {
    if (decltype(st)::value < nk) issue(st, decltype(st)::value);
  });
  if (nk >= S - 1) wait_vmcnt<(S - 2) * L>();
  else wait_vmcnt<0>();
  barrier_no_fence();
  // iteration i refills the stage of tile i - 1 (free since the last barrier)
  // with tile i + S - 1, multiplies stage i % S, then waits for tile i + 1.
  // The loop body is U rounds of the ring: at the loop head the compiler's
  // wait-count tracking merges both paths and waits for every load in flight,
  // so a longer body drains the pipeline less often.
  for (int it = 0; it < nk; it += S * U) {
    static_for<0, S * U>([&](auto du) {
      constexpr int dd = decltype(du)::value % S;
      const int i = it + decltype(du)::value;
      if (i >= nk) return;
      // the guard around each load also keeps the scheduler from gathering them
      const bool more = i + S - 1 < nk;
      compute(std::integral_constant<int, dd>{}, [&](auto qc) {
        static_for<0, L>([&](auto hc) {
          if constexpr (slot(decltype(hc)::value) == decltype(qc)::value) {
            if (more) issue_one(std::integral_constant<int, (dd + S - 1) % S>{}, i + S - 1, hc);
          }
        });
      });
      if (more) wait_ring<(S - 2) * L>();
      else wait_ring<0>();
      barrier_no_fence();
    });
  }
  if constexpr (STAGED) {
    // every wave is past the last barrier, so the ring is free
    static_assert(WTN == 64, "staging rows are 128 bytes");
    constexpr int WB = WTM * WTN;  // elements per wave
    static_assert(NW * WB <= S * ST, "staging fits in the ring");
    const int off = wave * WB;
    uint16_t *stg = off < ST ? T0 + off : off < 2 * ST ? T1 + (off - ST) : off < 3 * ST ? T2 + (off - 2 * ST)
                                                                                           : T3 + (off - 3 * ST);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = 32 * i + fr;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // columns 32j + 8q + 4fh .. +3 of row r: half of 16-byte chunk 4j + q
          const int chunk = (4 * j + q) ^ (r & 7);
          uint2 v;
          v.x = uint32_t(f32_to_bf16(acc[i][j][4 * q])) | (uint32_t(f32_to_bf16(acc[i][j][4 * q + 1])) << 16);
          v.y = uint32_t(f32_to_bf16(acc[i][j][4 * q + 2])) | (uint32_t(f32_to_bf16(acc[i][j][4 * q + 3])) << 16);
          *reinterpret_cast<uint2 *>(stg + r * WTN + chunk * 8 + 4 * fh) = v;
        }
    }
    // the staged rows are this wave's own: LDS operations of one wave complete in order
#pragma unroll
    for (int t = 0; t < WB / 8 / 64; ++t) {
      const int idx = t * 64 + lane, r = idx >> 3, c = idx & 7;
      const uint4 v = *reinterpret_cast<const uint4 *>(stg + r * WTN + (c ^ (r & 7)) * 8);
      const int row = row0 + wm + r, col = col0 + wn + 8 * c;
      if (row < M && col < N)
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(C) + static_cast<int64_t>(row) * ldc + col) = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = col0 + wn + 32 * j + fr;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + wm + 32 * i + 8 * (r >> 2) + 4 * fh + (r & 3);
          if (row >= M) continue;
          const int64_t o = static_cast<int64_t>(row) * ldc + col;
          if (CBF16)
            static_cast<uint16_t *>(C)[o] = f32_to_bf16(acc[i][j][r]);
          else
            static_cast<float *>(C)[o] = acc[i][j][r];
        }
      }
  }
}

// bf16 split-K product of two row-major operands over their rows (the weight
// gradients sum over edges, and the edge index is the rows of both dY and the
// saved GEMM input).  The tiles go to LDS as they lie in memory, [k][m] and
// [k][n], 512-byte rows (BM = BN = 256), by the same direct loads and ring as
// gemm_bf16_lds_kernel; MFMA fragments need eight consecutive k of one m, which
// gfx950's transposing LDS read (ds_read_b64_tr_b16) delivers: within each
// group of 16 lanes, lane i receives element i % 4 of the 8-byte reads of
// lanes i / 4 + 4 j, j = 0..3.  So lanes 4q..4q+3 of a group read 32
// consecutive bytes of row k0 + q, and lane i gets k0..k0+3 of column
// base + i; two such reads (k0 and k0 + 4) make one bf16x8 fragment.  The
// 16-byte chunks of row k are XOR-swizzled by tn_swizzle(k), which puts the
// rows read together on distinct LDS banks.  Rows past the end of the K range
// are read from a block of zeros.
__device__ __align__(16) uint16_t g_zero_row[512] = {0};

__device__ inline int tn_swizzle(int k) { return ((k & 3) << 2) | (((k >> 3) & 1) << 4); }

template <int BK, int WM, int WN, int S>
__global__ void __launch_bounds__(64 * WM * WN, 1) gemm_bf16_tn_kernel(int M, int N, int K,
                                                                     const uint16_t *__restrict__ P, int ldp,
                                                                     const uint16_t *__restrict__ Q, int ldq,
                                                                     float *__restrict__ C, int ldc, int splits,
                                                                     int k_per_split, int64_t split_stride) {
  constexpr int BM = 256, BN = 256, NW = WM * WN, ST = (BM + BN) * BK;
  static_assert(S == 2, "two-stage ring");
  __shared__ uint16_t T0[ST], T1[ST];
  // see gemm_bf16_lds_kernel: an unexecuted direct load placed first
  __shared__ __attribute__((aligned(1024))) uint32_t dma_anchor[256];
  if (K < 0) __builtin_amdgcn_global_load_lds(static_cast<const void *>(P), static_cast<void *>(dma_anchor), 16, 0, 0);
  auto ts = [&](auto st) -> uint16_t * {
    if constexpr (decltype(st)::value == 0) return T0;
    else return T1;
  };
  auto ps = [&](auto st) -> uint16_t * { return ts(st); };
  auto qs = [&](auto st) -> uint16_t * { return ts(st) + BK * BM; };
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const TileMap tm = map_tile(blockIdx.x, tiles_m, tiles_n, splits);
  if (!tm.valid) return;
  const int k_begin = tm.z * k_per_split, k_end = min(K, k_begin + k_per_split);
  const int nk = max(0, k_end - k_begin + BK - 1) / BK;
  C += tm.z * split_stride;
  const int row0 = tm.mt * BM, col0 = tm.nt * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  const int wm = (wave / WN) * WTM, wn = (wave % WN) * WTN;
  // direct loads: a BK x 32-chunk operand tile is BK / 2 wave loads (2 rows each), spread over the waves
  constexpr int LA = BK * 32 / 64 / NW;
  static_assert(LA >= 1 && (BK * 32) % (64 * NW) == 0, "tile");
  int lrow[LA], lcol[LA], loff[LA];
#pragma unroll
  for (int h = 0; h < LA; ++h) {
    const int slot0 = (h * NW + wave) * 64, sl = slot0 + lane, r = sl >> 5;
    lrow[h] = r;
    lcol[h] = ((sl & 31) ^ tn_swizzle(r)) * 8;  // first column of the chunk this lane fetches
    loff[h] = slot0 * 8;
  }
  // direct load h of a K-tile: h < LA from P, then LA from Q.  Columns past M
  // (N) repeat the last chunk (those rows and columns of C are not written);
  // rows past the K range read zeros.
  auto issue_one = [&](auto st, int kt, auto hc) {
    constexpr int h = decltype(hc)::value % LA;
    constexpr bool from_q = decltype(hc)::value >= LA;
    const int k = k_begin + kt * BK + lrow[h];
    const bool in = k < k_end;
    const uint16_t *g = from_q ? (in ? Q + static_cast<int64_t>(k) * ldq + min(col0 + lcol[h], N - 8) : g_zero_row + lcol[h])
                               : (in ? P + static_cast<int64_t>(k) * ldp + min(row0 + lcol[h], M - 8) : g_zero_row + lcol[h]);
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(g), static_cast<void *>((from_q ? qs(st) : ps(st)) + loff[h]),
                                     16, 0, 0);
  };
  auto issue = [&](auto st, int kt) {
    static_for<0, 2 * LA>([&](auto hc) { issue_one(st, kt, hc); });
  };
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int grp = lane >> 4, gl = lane & 15;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  // fragment of columns base..base+31 and k = kk..kk+15 of an LDS tile (lane: column base + lane % 32,
  // k = kk + 8 (lane / 32) .. + 7)
  auto frag = [&](const uint16_t *tile, int base, int kk) -> bf16x8 {
    u32x2 h[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = kk + 8 * (grp >> 1) + 4 * u + (gl >> 2);
      const int col = base + 16 * (grp & 1) + 4 * (gl & 3);
      const int off = k * BM + (((col >> 3) ^ tn_swizzle(k)) << 3) + (col & 7);
      h[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                           (__attribute__((address_space(3))) s16x4 *)(tile + off)));
    }
    // whole dwords: element-wise assembly was seen to drop half of each read
    const u32x4 w = {h[0].x, h[0].y, h[1].x, h[1].y};
    return __builtin_bit_cast(bf16x8, w);
  };
  auto load_frag = [&](auto st, int s, bf16x8(&a)[TM], bf16x8(&b)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = frag(ps(st), wm + 32 * i, 16 * s);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = frag(qs(st), wn + 32 * j, 16 * s);
  };
  // hook(q) runs before the q-th MFMA of the K-tile
  auto mma = [&](bf16x8(&a)[TM], bf16x8(&b)[TN], auto sc, auto &&hook) {
    static_for<0, TM * TN>([&](auto qc) {
      constexpr int i = decltype(qc)::value / TN, j = decltype(qc)::value % TN;
      hook(std::integral_constant<int, decltype(sc)::value * TM * TN + decltype(qc)::value>{});
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    });
  };
  // fragments of k-step s + 1 are read while step s multiplies
  auto compute = [&](auto st, auto &&hook) {
    bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
    load_frag(st, 0, a0, b0);
    __builtin_amdgcn_s_setprio(1);  // the products issue ahead of the other wave's memory work
    static_for<0, BK / 16>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s % 2 == 0) {
        if constexpr (s + 1 < BK / 16) load_frag(st, s + 1, a1, b1);
        mma(a0, b0, sc, hook);
      } else {
        if constexpr (s + 1 < BK / 16) load_frag(st, s + 1, a0, b0);
        mma(a1, b1, sc, hook);
      }
    });
    __builtin_amdgcn_s_setprio(0);
  };
  // ring of two stages; the next K-tile's loads go out one at a time between
  // the products of the first half of the current one (see gemm_bf16_lds_kernel)
  constexpr int L = 2 * LA, NMF = TM * TN * (BK / 16);
  auto slot = [](int h) { return h * (NMF / 2) / L; };
  if (nk > 0) issue(std::integral_constant<int, 0>{}, 0);
  wait_vmcnt<0>();
  barrier_no_fence();
  for (int it = 0; it < nk; it += 2) {
    static_for<0, 2>([&](auto du) {
      constexpr int dd = decltype(du)::value;
      const int i = it + dd;
      if (i >= nk) return;
      const bool more = i + 1 < nk;
      compute(std::integral_constant<int, dd>{}, [&](auto qc) {
        static_for<0, L>([&](auto hc) {
          if constexpr (slot(decltype(hc)::value) == decltype(qc)::value) {
            if (more) issue_one(std::integral_constant<int, 1 - dd>{}, i + 1, hc);
          }
        });
      });
      wait_ring<0>();
      barrier_no_fence();
    });
  }
  const int fr = lane & 31, fh = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = col0 + wn + 32 * j + fr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm + 32 * i + 8 * (r >> 2) + 4 * fh + (r & 3);
        if (row < M) C[static_cast<int64_t>(row) * ldc + col] = acc[i][j][r];
      }
    }
}

}  // namespace

namespace {

// 128-wide tiles (2 MFMA tiles per wave) unless they would pad the dimension
// by more than 10% and 64-wide ones pad less (192 and 320 here).
int tile_count(int n) {
  const int r128 = (n + 127) / 128 * 128, pad128 = r128 - n, pad64 = (n + 63) / 64 * 64 - n;
  return (pad64 < pad128 && 10 * pad128 > r128) ? 1 : 2;
}

template <bool AK, bool BK_>
void launch_gemm(int tmt, int tnt, int M, int N, int K, const float *A, int lda, const float *B, int ldb, float *C,
                 int ldc, int splits, int kps, int64_t split_stride, hipStream_t stream) {
  const int tiles = ((M + 64 * tmt - 1) / (64 * tmt)) * ((N + 64 * tnt - 1) / (64 * tnt));
  const int grid = tile_grid(tiles, splits);
#define EGNN_G(TM_, TN_) \
  gemm_f32_kernel<AK, BK_, TM_, TN_><<<grid, 256, 0, stream>>>(M, N, K, A, lda, B, ldb, C, ldc, splits, kps, split_stride)
  if (tmt == 2 && tnt == 2) EGNN_G(2, 2);
  else if (tmt == 2) EGNN_G(2, 1);
  else if (tnt == 2) EGNN_G(1, 2);
  else EGNN_G(1, 1);
#undef EGNN_G
}

template <bool UK, bool VK, bool PRE>
void launch_cgemm(int tmt, int tnt, int M, int N, int K, const float *Up, const float *Um, int ldu, const float *V1,
                  const float *V2, const float *V3, int ldv, float vsign, float *Cre, float *Cim, int ldc, int splits,
                  int kps, int64_t split_stride, hipStream_t stream) {
  const int tiles = ((M + 64 * tmt - 1) / (64 * tmt)) * ((N + 64 * tnt - 1) / (64 * tnt));
  const int grid = tile_grid(tiles, splits);
#define EGNN_C(TM_, TN_)                                                                                           \
  cgemm_f32_kernel<UK, VK, PRE, TM_, TN_><<<grid, 256, 0, stream>>>(M, N, K, Up, Um, ldu, V1, V2, V3, ldv, vsign, Cre, \
                                                                    Cim, ldc, splits, kps, split_stride)
  if (tmt == 2 && tnt == 2) EGNN_C(2, 2);
  else if (tmt == 2) EGNN_C(2, 1);
  else if (tnt == 2) EGNN_C(1, 2);
  else EGNN_C(1, 1);
#undef EGNN_C
}

}  // namespace

int gemm_f32_tiles(int M, int N) {
  const int tmt = tile_count(M), tnt = tile_count(N);
  return ((M + 64 * tmt - 1) / (64 * tmt)) * ((N + 64 * tnt - 1) / (64 * tnt));
}

int gemm_bf16_tn_tiles(int M, int N) { return ((M + 255) / 256) * ((N + 255) / 256); }

namespace {
template <typename F>
int blocks_per_cu(F kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(kernel), threads, 0) !=
          hipSuccess ||
      n < 1)
    n = 1;
  return n;
}
}  // namespace

int gemm_f32_tn_blocks_per_cu(int M, int N) {
  static const int o[4] = {blocks_per_cu(gemm_f32_kernel<false, false, 1, 1>, 256),
                           blocks_per_cu(gemm_f32_kernel<false, false, 1, 2>, 256),
                           blocks_per_cu(gemm_f32_kernel<false, false, 2, 1>, 256),
                           blocks_per_cu(gemm_f32_kernel<false, false, 2, 2>, 256)};
  return o[(tile_count(M) - 1) * 2 + (tile_count(N) - 1)];
}

int cgemm_f32_dw_blocks_per_cu(int M, int N) {
  static const int o[4] = {blocks_per_cu(cgemm_f32_kernel<false, false, false, 1, 1>, 256),
                           blocks_per_cu(cgemm_f32_kernel<false, false, false, 1, 2>, 256),
                           blocks_per_cu(cgemm_f32_kernel<false, false, false, 2, 1>, 256),
                           blocks_per_cu(cgemm_f32_kernel<false, false, false, 2, 2>, 256)};
  return o[(tile_count(M) - 1) * 2 + (tile_count(N) - 1)];
}

int gemm_bf16_tn_blocks_per_cu() {
  static const int o = blocks_per_cu(gemm_bf16_tn_kernel<64, 2, 4, 2>, 512);
  return o;
}

int xcd_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || n < kXcd)
    return 32;
  return n / kXcd;
}

hipError_t gemm_f32(int M, int N, int K, const float *A, int lda, bool a_kcontig, const float *B, int ldb,
                    bool b_kcontig, float *C, int ldc, int splits, int64_t split_stride, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (splits < 1) splits = 1;
  int kps = (K + splits - 1) / splits;
  kps = (kps + BK - 1) / BK * BK;
  const int tmt = tile_count(M), tnt = tile_count(N);
  if (a_kcontig && b_kcontig)
    launch_gemm<true, true>(tmt, tnt, M, N, K, A, lda, B, ldb, C, ldc, splits, kps, split_stride, stream);
  else if (!a_kcontig && !b_kcontig)
    launch_gemm<false, false>(tmt, tnt, M, N, K, A, lda, B, ldb, C, ldc, splits, kps, split_stride, stream);
  else if (a_kcontig)
    launch_gemm<true, false>(tmt, tnt, M, N, K, A, lda, B, ldb, C, ldc, splits, kps, split_stride, stream);
  else
    launch_gemm<false, true>(tmt, tnt, M, N, K, A, lda, B, ldb, C, ldc, splits, kps, split_stride, stream);
  return hipGetLastError();
}

hipError_t cgemm_f32(int M, int N, int K, const float *Up, const float *Um, int ldu, bool u_kcontig, const float *V1,
                     const float *V2, const float *V3, int ldv, bool v_kcontig, float vsign, float *Cre, float *Cim,
                     int ldc, int splits, int64_t split_stride, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (splits < 1) splits = 1;
  int kps = (K + splits - 1) / splits;
  kps = (kps + CBK - 1) / CBK * CBK;
  const int tmt = tile_count(M), tnt = tile_count(N);
  const bool pre = V3 != nullptr;
  if (u_kcontig && v_kcontig && pre)
    launch_cgemm<true, true, true>(tmt, tnt, M, N, K, Up, Um, ldu, V1, V2, V3, ldv, vsign, Cre, Cim, ldc, splits, kps,
                                   split_stride, stream);
  else if (u_kcontig && !v_kcontig && pre)
    launch_cgemm<true, false, true>(tmt, tnt, M, N, K, Up, Um, ldu, V1, V2, V3, ldv, vsign, Cre, Cim, ldc, splits, kps,
                                    split_stride, stream);
  else if (!u_kcontig && !v_kcontig && !pre)
    launch_cgemm<false, false, false>(tmt, tnt, M, N, K, Up, Um, ldu, V1, V2, V3, ldv, vsign, Cre, Cim, ldc, splits,
                                      kps, split_stride, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

namespace {

hipError_t launch_bf16(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B, int ldb, void *C, int ldc,
                       bool c_bf16, int splits, int64_t split_stride, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % 8 != 0 || lda % 8 != 0 || ldb % 8 != 0) return hipErrorInvalidValue;
  const bool aligned = (reinterpret_cast<uintptr_t>(A) % 16 == 0) && (reinterpret_cast<uintptr_t>(B) % 16 == 0);
  const int waste256 = (N + 255) / 256 * 256 - N, waste128 = (N + 127) / 128 * 128 - N;
  const int tiles_m = (M + 255) / 256;
  // K per split: a multiple of the K tile
  auto kps_for = [&](int bk) { return ((K + splits - 1) / splits + bk - 1) / bk * bk; };
  // bf16 output written through LDS as 16-byte rows (see gemm_bf16_lds_kernel)
  const bool staged = c_bf16 && N % 8 == 0 && ldc % 8 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0;
#define EGNN_B(BM_, BN_, BK_, WM_, WN_, S_, U_)                                                                    \
  do {                                                                                                          \
    const int grid = tile_grid(tiles_m * ((N + BN_ - 1) / BN_), splits);                                        \
    const int kps = kps_for(BK_);                                                                               \
    if (staged)                                                                                                 \
      gemm_bf16_lds_kernel<BM_, BN_, BK_, WM_, WN_, S_, U_, true, true>                                         \
          <<<grid, 64 * WM_ * WN_, 0, stream>>>(M, N, K, A, lda, B, ldb, C, ldc, splits, kps, split_stride);    \
    else if (c_bf16)                                                                                            \
      gemm_bf16_lds_kernel<BM_, BN_, BK_, WM_, WN_, S_, U_, true, false>                                        \
          <<<grid, 64 * WM_ * WN_, 0, stream>>>(M, N, K, A, lda, B, ldb, C, ldc, splits, kps, split_stride);    \
    else                                                                                                        \
      gemm_bf16_lds_kernel<BM_, BN_, BK_, WM_, WN_, S_, U_, false, false>                                       \
          <<<grid, 64 * WM_ * WN_, 0, stream>>>(M, N, K, A, lda, B, ldb, C, ldc, splits, kps, split_stride);    \
  } while (0)
  if (aligned && K % 64 == 0 && waste128 < waste256) {
    // 256 x 128 x 64, 8 waves (4 x 2, 64 x 64 each), 3 stages (144 KB LDS): N = 640 and the like;
    // loop body of two ring rounds
    EGNN_B(256, 128, 64, 4, 2, 3, 2);
  } else if (aligned && K % 64 == 0) {
    // 256 x 256 x 64, 8 waves (2 x 4, 128 x 64 each), 2 stages (128 KB LDS): 128-byte rows per load;
    // loop body of four ring rounds (eight K-tiles: 0.5-2.5% faster than four on the layer's shapes)
    EGNN_B(256, 256, 64, 2, 4, 2, 4);
  } else if (aligned && K % 32 == 0) {
    // 256 x 256 x 32, 4 stages (128 KB LDS), loop body of 4 rings
    EGNN_B(256, 256, 32, 2, 4, 4, 4);
#undef EGNN_B
  } else {
    if (splits != 1) return hipErrorInvalidValue;
    const int tiles = ((M + HBM_ - 1) / HBM_) * ((N + HBN - 1) / HBN);
    const int grid = tile_grid(tiles, 1);
    if (c_bf16)
      gemm_bf16_kernel<true><<<grid, 256, 0, stream>>>(M, N, K, A, lda, B, ldb, C, ldc);
    else
      gemm_bf16_kernel<false><<<grid, 256, 0, stream>>>(M, N, K, A, lda, B, ldb, C, ldc);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16_nt(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B, int ldb, void *C, int ldc,
                        bool c_bf16, hipStream_t stream) {
  return launch_bf16(M, N, K, A, lda, B, ldb, C, ldc, c_bf16, 1, 0, stream);
}

hipError_t gemm_bf16_nt_splitk(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B, int ldb, float *C,
                               int ldc, int splits, int64_t split_stride, hipStream_t stream) {
  if (splits < 1) splits = 1;
  if (K % 32 != 0) return hipErrorInvalidValue;
  return launch_bf16(M, N, K, A, lda, B, ldb, C, ldc, false, splits, split_stride, stream);
}

hipError_t gemm_bf16_tn_splitk(int M, int N, int K, const uint16_t *P, int ldp, const uint16_t *Q, int ldq, float *C,
                               int ldc, int splits, int64_t split_stride, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (splits < 1) splits = 1;
  if (M % 8 != 0 || N % 8 != 0 || ldp % 8 != 0 || ldq % 8 != 0 || K < 0 ||
      reinterpret_cast<uintptr_t>(P) % 16 != 0 || reinterpret_cast<uintptr_t>(Q) % 16 != 0)
    return hipErrorInvalidValue;
  constexpr int BK = 64;
  int kps = (K + splits - 1) / splits;
  kps = (kps + BK - 1) / BK * BK;
  const int grid = tile_grid(((M + 255) / 256) * ((N + 255) / 256), splits);
  // 256 x 256 x 64, 8 waves (2 x 4, 128 x 64 each), 2 stages (128 KB LDS)
  gemm_bf16_tn_kernel<BK, 2, 4, 2><<<grid, 512, 0, stream>>>(M, N, K, P, ldp, Q, ldq, C, ldc, splits, kps, split_stride);
  return hipGetLastError();
}

}  // namespace egnn
