// Expert path for large batches (prefill): the gate/up and down projections
// of the activated experts as bf16 MFMA grouped GEMMs, plus an MFMA router.
//
// The layer ("Paper of the Week #3 - Half the FLOPs Is Not Half the Time",
// section "The Receipt", Eq. 2 for the weights; "Channel Selection for
// Mixture-of-Experts Decoding Needs No Calibration Data", section 2
// "Background" for the gated-MLP experts): for the tokens routed to expert e,
//   A_e = x[tokens of e]                       [n_e, H]  bf16
//   a   = silu(A_e Wg[e]^T) * (A_e Wu[e]^T) * w  [n_e, I] -> bf16
//   z   = a Wd[e]^T                             [n_e, H]  fp32 -> bf16
// and y[t] = sum of z over the token's k1 slots, in slot order, in fp32.
//
// Every product is "NT": both operands are stored K-contiguous (x and a rows
// along H / I, weight rows along H / I), which is the layout the MFMA
// operands want.  One tile engine serves all three GEMMs:
//   block = 256 threads = 4 waves in a 2x2 grid, tile BM x BN (128 x 128 for
//   the expert GEMMs, 64 x 64 for the router), K step 64 bf16; each wave owns
//   a (BM/2) x (BN/2) sub-tile of MFMA 32x32x16 (v_mfma_f32_32x32x16_bf16)
//   accumulators; A and B K-slices are staged in LDS (double buffered, rows
//   padded by 16 bytes), the next slice's global loads are in flight while
//   the current one is multiplied.
// Lane layouts of v_mfma_f32_32x32x16_bf16 (checked on the device): lane l
// holds A row l%32 and B column l%32, k = 8*(l/32) .. +7; accumulator r of
// lane l is row (r/4)*8 + (l/32)*4 + r%4, column l%32.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace pf {

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int LDS_ROW = BK + 8;  // bf16 elements per LDS row (16-byte pad)
constexpr int GM = 128, GN = 128;  // tile of the expert GEMMs

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int BM, int BN>
struct Tile {
  uint16_t a[2][BM][LDS_ROW];
  uint16_t b[2][BN][LDS_ROW];
};

// One K slice of A (BM x BK) and B (BN x BK) is BM*8 + BN*8 chunks of 16 B;
// chunk i*256 + t of an operand is row i*32 + t/8, k offset (t%8)*8, so eight
// consecutive threads read one row's 128 contiguous bytes.
template <int BM, int BN>
struct Loader {
  static constexpr int NA = BM / 32, NB = BN / 32;
  const uint16_t *arow[NA];
  const uint16_t *brow[NB];
  uint4 ra[NA], rb[NB];

  __device__ static int row(int i) { return i * 32 + (threadIdx.x >> 3); }
  __device__ void fetch(int k0) {
    const int q = (threadIdx.x & 7) * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[i] = ld16(arow[i] + k0 + q);
#pragma unroll
    for (int j = 0; j < NB; ++j) rb[j] = ld16_stream(brow[j] + k0 + q);
  }
  __device__ void store(Tile<BM, BN> &T, int buf) {
    const int q = (threadIdx.x & 7) * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<uint4 *>(&T.a[buf][row(i)][q]) = ra[i];
#pragma unroll
    for (int j = 0; j < NB; ++j) *reinterpret_cast<uint4 *>(&T.b[buf][row(j)][q]) = rb[j];
  }
  // the same through an explicit register stage (several slices in flight)
  struct Stage {
    uint4 a[NA], b[NB];
  };
  __device__ void fetch(int k0, Stage &r) const {
    const int q = (threadIdx.x & 7) * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) r.a[i] = ld16(arow[i] + k0 + q);
#pragma unroll
    for (int j = 0; j < NB; ++j) r.b[j] = ld16_stream(brow[j] + k0 + q);
  }
  __device__ static void store(Tile<BM, BN> &T, int buf, const Stage &r) {
    const int q = (threadIdx.x & 7) * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<uint4 *>(&T.a[buf][row(i)][q]) = r.a[i];
#pragma unroll
    for (int j = 0; j < NB; ++j) *reinterpret_cast<uint4 *>(&T.b[buf][row(j)][q]) = r.b[j];
  }
};

// acc[i][j] += A(wave rows i) * B(wave cols j)^T over one K slice in LDS;
// the 2x2 waves own (BM/2) x (BN/2) sub-tiles of 32x32 MFMA blocks.
template <int BM, int BN>
__device__ __forceinline__ void mma_slice(const Tile<BM, BN> &T, int buf, int wm, int wn,
                                          f32x16_t (&acc)[BM / 64][BN / 64]) {
  constexpr int MI = BM / 64, NI = BN / 64;
  const int l = lane_id();
  const int lr = l & 31, lk = (l >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < BK; ks += 16) {
    bf16x8_t af[MI], bf[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      af[i] = *reinterpret_cast<const bf16x8_t *>(&T.a[buf][wm * (BM / 2) + i * 32 + lr][ks + lk]);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      bf[j] = *reinterpret_cast<const bf16x8_t *>(&T.b[buf][wn * (BN / 2) + j * 32 + lr][ks + lk]);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
  }
}

// Full K loop, double buffered in LDS: the next slice's global loads are in
// flight while the current slice is multiplied.  K is a multiple of BK.
template <int BM, int BN, typename LD>
__device__ void mma_k_loop(Tile<BM, BN> &T, LD &ld, int K, int wm, int wn,
                           f32x16_t (&acc)[BM / 64][BN / 64]) {
  const int nk = K / BK;
  ld.fetch(0);
  ld.store(T, 0);
  __syncthreads();
  for (int kk = 0; kk < nk; ++kk) {
    const int buf = kk & 1;
    if (kk + 1 < nk) ld.fetch((kk + 1) * BK);
    mma_slice<BM, BN>(T, buf, wm, wn, acc);
    if (kk + 1 < nk) ld.store(T, buf ^ 1);
    __syncthreads();
  }
}

// The K loop for a K known at compile time (NK slices), fully unrolled: the
// slices stream through a ring of kStages register stages into the two LDS
// buffers, so that while slice k is multiplied out of LDS the loads of
// slices k+1 .. k+kStages are in flight, and slice k+1 is written to the
// other buffer once it has arrived.  Unrolled, every wait for a stage's
// loads leaves the younger stages' loads outstanding (in a rolled loop the
// compiler waited for every load at each store, which left one slice in
// flight whatever the ring).
constexpr int kStages = 3;

template <int BM, int BN, int NK, typename LD>
__device__ __forceinline__ void mma_k_loop_fixed(Tile<BM, BN> &T, LD &ld, int wm, int wn,
                                                 f32x16_t (&acc)[BM / 64][BN / 64]) {
  using Stage = typename LD::Stage;
  Stage ring[kStages];
#pragma unroll
  for (int q = 0; q < kStages; ++q)
    if (q < NK) ld.fetch(q * BK, ring[q]);
  LD::store(T, 0, ring[0]);
  if (kStages < NK) ld.fetch(kStages * BK, ring[0]);
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    mma_slice<BM, BN>(T, kk & 1, wm, wn, acc);
    if (kk + 1 < NK) LD::store(T, (kk + 1) & 1, ring[(kk + 1) % kStages]);
    if (kk + 1 + kStages < NK) ld.fetch((kk + 1 + kStages) * BK, ring[(kk + 1) % kStages]);
    __syncthreads();
  }
}

// K loop of the expert GEMMs: NK > 0 slices unrolled, NK = 0 the
// double-buffered loop over any K (a kernel instantiation per NK keeps each
// one's registers to itself).
template <int NK, int BM, int BN, typename LD>
__device__ __forceinline__ void mma_k_any(Tile<BM, BN> &T, LD &ld, int K, int wm, int wn,
                                          f32x16_t (&acc)[BM / 64][BN / 64]) {
  if constexpr (NK > 0)
    mma_k_loop_fixed<BM, BN, NK>(T, ld, wm, wn, acc);
  else
    mma_k_loop<BM, BN>(T, ld, K, wm, wn, acc);
}

// the K of the measured layers get an unrolled loop
__host__ __device__ constexpr int unrolled_nk(int K) {
  return (K == 768 || K == 1024 || K == 2048 || K == 4096) ? K / BK : 0;
}

template <int MI, int NI>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[MI][NI]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// row (within the BM-row tile) of accumulator element r of MFMA block (i, .)
template <int BM>
__device__ __forceinline__ int acc_row(int wm, int i, int r) {
  return wm * (BM / 2) + i * 32 + (r >> 2) * 8 + (lane_id() >> 5) * 4 + (r & 3);
}

// ------------------------------------------------------------------ plan
// plan layout (int32): [0] U, [1] total M tiles, [4 .. 4+E) uniq,
// off[E+1], mt_off[E+1] (first M tile of each unique expert), list[n].
// Assignments of one expert appear in the order the atomic scatter gives;
// each GEMM row is computed independently of its position, so y does not
// depend on that order.
constexpr int kPlanPer = 16;
constexpr int kPlanStage = 32768;  // 128 KB of LDS

__global__ __launch_bounds__(1024) void prefill_plan_kernel(const int32_t *__restrict__ ids,
                                                            int64_t n, int E,
                                                            int32_t *__restrict__ plan) {
  __shared__ int32_t cnt[kMaxExperts], uidx[kMaxExperts], fill[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t wsum[16][3];
  // up to kPlanStage assignments are scattered in LDS and written out
  // coalesced: scattered 4-byte global stores from one workgroup are slow
  __shared__ int32_t s_list[kPlanStage];
  const bool staged = n <= kPlanStage;
  int32_t *uniq = plan + 4;
  int32_t *off = uniq + E;
  int32_t *mt_off = off + E + 1;
  int32_t *list = mt_off + E + 1;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  for (int e = tid; e < E; e += 1024) {
    cnt[e] = 0;
    fill[e] = 0;
  }
  __syncthreads();
  // ids are read kPlanPer per thread at a time, all loads issued before the
  // LDS atomics that consume them
  for (int64_t b = 0; b < n; b += (int64_t)1024 * kPlanPer) {
    int32_t ev[kPlanPer];
#pragma unroll
    for (int q = 0; q < kPlanPer; ++q) {
      const int64_t i = b + (int64_t)q * 1024 + tid;
      ev[q] = i < n ? ids[i] : -1;
    }
#pragma unroll
    for (int q = 0; q < kPlanPer; ++q)
      if (ev[q] >= 0) atomicAdd(&cnt[ev[q]], 1);
  }
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  int v[3] = {c > 0 ? 1 : 0, c, (c + GM - 1) / GM};
  int inc[3] = {v[0], v[1], v[2]};
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int t = __shfl_up(inc[q], o);
      if (lane >= o) inc[q] += t;
    }
  }
  if (lane == kWave - 1)
    for (int q = 0; q < 3; ++q) wsum[wv][q] = inc[q];
  __syncthreads();
  int base[3] = {0, 0, 0};
  for (int k = 0; k < wv; ++k)
    for (int q = 0; q < 3; ++q) base[q] += wsum[k][q];
  const int ex_u = base[0] + inc[0] - v[0];
  const int ex_c = base[1] + inc[1] - v[1];
  const int ex_m = base[2] + inc[2] - v[2];
  if (tid < E) {
    uidx[tid] = ex_u;
    if (c > 0) {
      uniq[ex_u] = tid;
      off[ex_u] = ex_c;
      s_off[ex_u] = ex_c;
      mt_off[ex_u] = ex_m;
    }
  }
  if (tid == 1023) {
    const int U = base[0] + inc[0];
    plan[0] = U;
    plan[1] = base[2] + inc[2];
    off[U] = (int32_t)n;
    mt_off[U] = base[2] + inc[2];
  }
  __syncthreads();
  for (int64_t b = 0; b < n; b += (int64_t)1024 * kPlanPer) {
    int32_t ev[kPlanPer];
#pragma unroll
    for (int q = 0; q < kPlanPer; ++q) {
      const int64_t i = b + (int64_t)q * 1024 + tid;
      ev[q] = i < n ? ids[i] : -1;
    }
#pragma unroll
    for (int q = 0; q < kPlanPer; ++q) {
      if (ev[q] >= 0) {
        const int pos = atomicAdd(&fill[ev[q]], 1);
        const int32_t i = (int32_t)(b + (int64_t)q * 1024 + tid);
        if (staged)
          s_list[s_off[uidx[ev[q]]] + pos] = i;
        else
          list[s_off[uidx[ev[q]]] + pos] = i;
      }
    }
  }
  if (staged) {
    __syncthreads();
    for (int i = tid; i < (int)n; i += 1024) list[i] = s_list[i];
  }
}

// Work tile j of the G = (M tiles) x NT tiles of a grouped GEMM, ordered
// (unique expert u, N tile, M tile of u): the M tiles of one expert that
// share an N tile (the same weight rows) are consecutive.  Blocks are handed
// to the 8 XCDs round-robin by index, so block b runs on XCD b % 8; XCD x
// takes the contiguous range of j starting at x * ceil(G / 8), and tiles
// that share weight rows run together on one XCD and share them through its
// L2.  Returns false for blocks beyond G.
__device__ bool tile_of(int b, const int32_t *mt_off, int U, int n_mt, int NT, int *u_out,
                        int *nt_out, int *mt_out) {
  const int G = n_mt * NT;
  const int per = (G + 7) / 8;
  const int slot = b >> 3, j = (b & 7) * per + slot;
  if (slot >= per || j >= G) return false;
  int lo = 0, hi = U - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mt_off[mid] * NT <= j)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int r = j - mt_off[lo] * NT;
  const int nmt = mt_off[lo + 1] - mt_off[lo];
  *u_out = lo;
  *nt_out = r / nmt;
  *mt_out = mt_off[lo] + r % nmt;
  return true;
}

// ------------------------------------------------------------------ gate/up
// Tile (M tile of expert u, 64 channels c0..c0+63).  B rows interleave gate
// and up: rows [64g, 64g+32) = Wg[e, c0+32g ..], rows [64g+32, 64g+64) =
// Wu[e, c0+32g ..]; wave (wm, wn) then holds the gate and the up value of
// the same (row, channel) in acc[i][0] and acc[i][1] of the same lane.
template <int NK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gateup_mma_kernel(
    const uint16_t *__restrict__ x, int H, const uint16_t *__restrict__ Wg,
    const uint16_t *__restrict__ Wu, int I, const int32_t *__restrict__ plan, int E, int k1,
    const float *__restrict__ w, uint16_t *__restrict__ abf) {
  __shared__ Tile<GM, GN> T;
  const int U = plan[0];
  const int32_t *uniq = plan + 4;
  const int32_t *off = uniq + E;
  const int32_t *mt_off = off + E + 1;
  const int32_t *list = mt_off + E + 1;
  int u, nt, mt;
  if (!tile_of(blockIdx.x, mt_off, U, plan[1], I / 64, &u, &nt, &mt)) return;
  const int e = uniq[u];
  const int lb = off[u], n_e = off[u + 1] - lb;
  const int row0 = (mt - mt_off[u]) * GM;
  const int c0 = nt * 64;
  const int tid = threadIdx.x, wv = tid >> 6, wm = wv >> 1, wn = wv & 1;
  Loader<GM, GN> ld;
#pragma unroll
  for (int i = 0; i < Loader<GM, GN>::NA; ++i) {
    const int m = min(row0 + Loader<GM, GN>::row(i), n_e - 1);
    ld.arow[i] = x + (int64_t)(list[lb + m] / k1) * H;
  }
#pragma unroll
  for (int j = 0; j < Loader<GM, GN>::NB; ++j) {
    const int rr = Loader<GM, GN>::row(j);
    const int g = rr >> 6, within = rr & 63;
    const int cc = c0 + g * 32 + (within & 31);
    ld.brow[j] = (within < 32 ? Wg : Wu) + ((int64_t)e * I + cc) * H;
  }
  f32x16_t acc[2][2];
  zero_acc(acc);
  mma_k_any<NK, GM, GN>(T, ld, H, wm, wn, acc);
  const int c = c0 + wn * 32 + (lane_id() & 31);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = row0 + acc_row<GM>(wm, i, r);
      if (m < n_e) {
        const int asg = list[lb + m];
        const float a = silu(acc[i][0][r]) * acc[i][1][r] * w[asg];
        abf[(int64_t)asg * I + c] = (uint16_t)f32_to_bf16_bits(a);
      }
    }
}

// ------------------------------------------------------------------ down
// Tile (M tile of expert u, 128 output rows h0..h0+127 of H):
// z[asg, h] = a[asg, :] . Wd[e, h, :], stored as bf16 (the layer's output is
// bf16; partials in bf16 halve the traffic of the slot combine).
template <int NK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_mma_kernel(
    const uint16_t *__restrict__ abf, int H, const uint16_t *__restrict__ Wd, int I,
    const int32_t *__restrict__ plan, int E, uint16_t *__restrict__ zbf) {
  __shared__ Tile<GM, GN> T;
  const int U = plan[0];
  const int32_t *uniq = plan + 4;
  const int32_t *off = uniq + E;
  const int32_t *mt_off = off + E + 1;
  const int32_t *list = mt_off + E + 1;
  int u, nt, mt;
  if (!tile_of(blockIdx.x, mt_off, U, plan[1], H / GN, &u, &nt, &mt)) return;
  const int e = uniq[u];
  const int lb = off[u], n_e = off[u + 1] - lb;
  const int row0 = (mt - mt_off[u]) * GM;
  const int h0 = nt * GN;
  const int tid = threadIdx.x, wv = tid >> 6, wm = wv >> 1, wn = wv & 1;
  Loader<GM, GN> ld;
#pragma unroll
  for (int i = 0; i < Loader<GM, GN>::NA; ++i) {
    const int m = min(row0 + Loader<GM, GN>::row(i), n_e - 1);
    ld.arow[i] = abf + (int64_t)list[lb + m] * I;
  }
#pragma unroll
  for (int j = 0; j < Loader<GM, GN>::NB; ++j)
    ld.brow[j] = Wd + ((int64_t)e * H + h0 + Loader<GM, GN>::row(j)) * I;
  f32x16_t acc[2][2];
  zero_acc(acc);
  mma_k_any<NK, GM, GN>(T, ld, I, wm, wn, acc);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = row0 + acc_row<GM>(wm, i, r);
      if (m < n_e) {
        const int asg = list[lb + m];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          zbf[(int64_t)asg * H + h0 + wn * 64 + j * 32 + (lane_id() & 31)] =
              (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
      }
    }
}

// ------------------------------------------------------------------ router
// fp32 router weights as three bf16 terms, Wr = W1 + W2 + W3 with
// W1 = bf16(Wr), W2 = bf16(Wr - W1), W3 = bf16(Wr - W1 - W2): 24 significant
// bits, i.e. the fp32 value (up to the last bit's rounding).  x is bf16, so
// every product is exact in fp32 and logits = (x W1^T + x W2^T) + x W3^T,
// each term accumulated in fp32.
__global__ void split_router_kernel(const float *__restrict__ Wr, int64_t n,
                                    uint16_t *__restrict__ w3) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = Wr[i];
  const uint32_t b1 = f32_to_bf16_bits(v);
  const float r1 = v - __uint_as_float(b1 << 16);
  const uint32_t b2 = f32_to_bf16_bits(r1);
  const float r2 = r1 - __uint_as_float(b2 << 16);
  const uint32_t b3 = f32_to_bf16_bits(r2);
  w3[i] = (uint16_t)b1;
  w3[n + i] = (uint16_t)b2;
  w3[2 * n + i] = (uint16_t)b3;
}

// Tile (64 tokens, 64 experts) of the router logits, all NT terms in one
// workgroup: B holds 64 * NT weight rows, placed so that wave (wm, wn)'s
// NT column blocks are the NT terms of the same 32 experts; accumulator
// acc[0][q] of a lane is then term q of the same (token, expert), and the
// terms are added in the fixed order above in registers (plus br).  With
// one term (a bf16 router weight, the router method on a bf16 model) the
// tile is the logits themselves, rounded to bf16.  Experts beyond E read a
// valid row and are not stored.
constexpr int RM = 64, RN = 64;

template <int NT, int NK>
__global__ __launch_bounds__(kThreads) void router_mma_kernel(const uint16_t *__restrict__ x,
                                                              int64_t T, int H,
                                                              const uint16_t *__restrict__ w3,
                                                              int E, const float *__restrict__ br,
                                                              float *__restrict__ logits,
                                                              float *__restrict__ logits2) {
  static_assert(NT == 1 || NT == 3, "one bf16 term or the split fp32 weight");
  constexpr int BN = RN * NT;
  __shared__ Tile<RM, BN> Tl;
  const int n_nt = (E + RN - 1) / RN;
  const int64_t mt = blockIdx.x / n_nt;
  const int nt = (int)(blockIdx.x - mt * n_nt);
  const int tid = threadIdx.x, wv = tid >> 6, wm = wv >> 1, wn = wv & 1;
  const int64_t t0 = mt * RM;
  const int e0 = nt * RN;
  f32x16_t acc[1][NT];
  zero_acc(acc);
  Loader<RM, BN> ld;
#pragma unroll
  for (int i = 0; i < Loader<RM, BN>::NA; ++i) {
    const int64_t t = min<int64_t>(t0 + Loader<RM, BN>::row(i), T - 1);
    ld.arow[i] = x + t * H;
  }
#pragma unroll
  for (int j = 0; j < Loader<RM, BN>::NB; ++j) {
    // B row r: wave column half r / (32 NT), term (r % (32 NT)) / 32
    const int r = Loader<RM, BN>::row(j);
    const int term = (r % (32 * NT)) / 32;
    const int e = min(e0 + (r / (32 * NT)) * 32 + (r & 31), E - 1);
    ld.brow[j] = w3 + (int64_t)term * E * H + (int64_t)e * H;
  }
  mma_k_any<NK, RM, BN>(Tl, ld, H, wm, wn, acc);
  const int e = e0 + wn * 32 + (lane_id() & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t t = t0 + acc_row<RM>(wm, 0, r);
    if (t < T && e < E) {
      float l;
      if constexpr (NT == 1) {
        l = round_bf16(acc[0][0][r]);
      } else {
        l = (acc[0][0][r] + acc[0][1][r]) + acc[0][2][r];
        if (br) l = l + br[e];
      }
      logits[t * E + e] = l;
      if (logits2) logits2[t * E + e] = l;
    }
  }
}

}  // namespace pf

bool prefill_supported(int H, int I, bool bf16) {
  return bf16 && H % pf::GN == 0 && I % 64 == 0 && H % pf::BK == 0 && I % pf::BK == 0;
}

size_t prefill_plan_words(int64_t n, int E) { return 4 + 3 * (size_t)E + 2 + (size_t)n; }

hipError_t launch_split_router(const float *Wr, int E, int H, uint16_t *w3, hipStream_t s) {
  const int64_t n = (int64_t)E * H;
  pf::split_router_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(Wr, n, w3);
  return hipGetLastError();
}

hipError_t launch_router_mma(const uint16_t *x, int64_t T, int H, const uint16_t *w3, int E,
                             int nterms, const float *br, float *logits, float *logits2,
                             hipStream_t s) {
  const int64_t tiles = ((T + pf::RM - 1) / pf::RM) * ((E + pf::RN - 1) / pf::RN);
#define RT(NT, NK) pf::router_mma_kernel<NT, NK><<<dim3((unsigned)tiles), dim3(pf::kThreads), 0, s>>>( \
    x, T, H, w3, E, br, logits, logits2)
  const int nk = pf::unrolled_nk(H);
  if (nterms == 1) {
    if (nk == 2048 / pf::BK) RT(1, 2048 / pf::BK);
    else if (nk == 4096 / pf::BK) RT(1, 4096 / pf::BK);
    else RT(1, 0);
  } else {
    if (nk == 2048 / pf::BK) RT(3, 2048 / pf::BK);
    else if (nk == 4096 / pf::BK) RT(3, 4096 / pf::BK);
    else RT(3, 0);
  }
#undef RT
  return hipGetLastError();
}

hipError_t launch_prefill_plan(const int32_t *ids, int64_t n, int E, int32_t *plan,
                               hipStream_t s) {
  pf::prefill_plan_kernel<<<1, 1024, 0, s>>>(ids, n, E, plan);
  return hipGetLastError();
}

// upper bound of the M tiles of a batch: one partial tile per expert; the
// grid is a multiple of 8 (one slot per XCD, see tile_of)
static int64_t max_mtiles(int64_t n, int E) {
  const int64_t u = n < E ? n : E;
  return (n + pf::GM - 1) / pf::GM + u;
}
static unsigned grouped_grid(int64_t tiles) { return (unsigned)(((tiles + 7) / 8) * 8); }

hipError_t launch_gateup_mma(const uint16_t *x, int H, const uint16_t *Wg, const uint16_t *Wu,
                             int I, const int32_t *plan, int E, int64_t n, int k1, const float *w,
                             uint16_t *abf, hipStream_t s) {
  const unsigned grid = grouped_grid(max_mtiles(n, E) * (I / 64));
#define GU(NK) pf::gateup_mma_kernel<NK><<<dim3(grid), dim3(pf::kThreads), 0, s>>>( \
    x, H, Wg, Wu, I, plan, E, k1, w, abf)
  switch (pf::unrolled_nk(H)) {
    case 2048 / pf::BK: GU(2048 / pf::BK); break;
    case 4096 / pf::BK: GU(4096 / pf::BK); break;
    default: GU(0);
  }
#undef GU
  return hipGetLastError();
}

hipError_t launch_down_mma(const uint16_t *abf, int H, const uint16_t *Wd, int I,
                           const int32_t *plan, int E, int64_t n, uint16_t *zbf, hipStream_t s) {
  const unsigned grid = grouped_grid(max_mtiles(n, E) * (H / pf::GN));
#define DN(NK) pf::down_mma_kernel<NK><<<dim3(grid), dim3(pf::kThreads), 0, s>>>( \
    abf, H, Wd, I, plan, E, zbf)
  switch (pf::unrolled_nk(I)) {
    case 768 / pf::BK: DN(768 / pf::BK); break;
    case 1024 / pf::BK: DN(1024 / pf::BK); break;
    default: DN(0);
  }
#undef DN
  return hipGetLastError();
}

// y[t, h] = sum over the token's k1 slots of z[t*k1 + r, h] (bf16 partials,
// fp32 sum in slot order); 8 outputs per thread with 16-byte accesses.
__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint16_t *__restrict__ zbf,
                                                           const uint16_t *__restrict__ zs,
                                                           int64_t T, int H, int k1,
                                                           uint16_t *__restrict__ y) {
  const int64_t i8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i8 >= T * H) return;
  const int64_t t = i8 / H, h = i8 - t * H;
  float s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) s[k] = 0.0f;
  for (int r = 0; r < k1; ++r) {
    float v[8];
    Elem<bf16_t>::widen(ld16(zbf + (t * k1 + r) * H + h), v);
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = s[k] + v[k];
  }
  if (zs) {
    float v[8];
    Elem<bf16_t>::widen(ld16(zs + t * H + h), v);
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = s[k] + v[k];
  }
  uint4 o;
  o.x = f32_to_bf16_bits(s[0]) | (f32_to_bf16_bits(s[1]) << 16);
  o.y = f32_to_bf16_bits(s[2]) | (f32_to_bf16_bits(s[3]) << 16);
  o.z = f32_to_bf16_bits(s[4]) | (f32_to_bf16_bits(s[5]) << 16);
  o.w = f32_to_bf16_bits(s[6]) | (f32_to_bf16_bits(s[7]) << 16);
  *reinterpret_cast<uint4 *>(y + i8) = o;
}

hipError_t launch_combine_bf16(const uint16_t *zbf, const uint16_t *zs, int64_t T, int H, int k1,
                               uint16_t *y, hipStream_t s) {
  const int64_t n8 = T * H / 8;
  combine_bf16_kernel<<<dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s>>>(zbf, zs, T, H, k1,
                                                                              y);
  return hipGetLastError();
}

}  // namespace moe
