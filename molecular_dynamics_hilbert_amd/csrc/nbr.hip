// nbr.hip -- neighbour-list rebuild on gfx950.
//
// The three levels of the Tessera abstract's neighbour search (space-filling-curve order,
// cells, pair filter with a conservative skin), as four stages:
//   1. wrap + 30-bit Hilbert key per atom (fp64, every operation rounded on its own),
//   2. stable LSD radix sort of (key, index), 4 passes of 8 bits; each 1024-key tile ranks
//      its keys with wave ballots (64 lanes) so equal digits keep their index order,
//   3. cell binning (cells at least (r_cut+skin)(1+1e-6) wide) into a cell-sorted copy of
//      the positions,
//   4. one block per cell stages its 27-cell stencil in LDS (sorted by (j, shift) for the
//      fill), and its waves test the cell's atoms against it: the fp64 pair test decides, the
//      wave compacts passing pairs with ballot + popcount, in row order. Count pass, scan,
//      fill pass.
// Decisions that must match the fp64 reference bit for bit are written with FP contraction
// off.
#include "tess_common.h"

#include <cstring>

#pragma clang fp contract(off)

namespace tess {
namespace {

constexpr int kMaxRow = 1024;
constexpr int kTile = 1024;  // radix-sort tile (256 threads x 4 rounds)

__device__ __forceinline__ float wrap_coord(float x, double L) {
  double t = (double)x / L;
  double f = floor(t);
  double p = f * L;
  double xw = (double)x - p;
  return (float)xw;
}

__device__ __forceinline__ uint32_t quant10(float xw, double L) {
  double S = 1024.0 / L;
  double v = floor((double)xw * S);
  v = v < 0.0 ? 0.0 : (v > 1023.0 ? 1023.0 : v);
  return (uint32_t)v;
}

// Skilling's transpose-form Hilbert index for 3 axes, 10 bits per axis; key bits are read
// level by level (most significant first), axis 0 first within a level.
__device__ __forceinline__ uint32_t hilbert30(uint32_t x0, uint32_t x1, uint32_t x2) {
  uint32_t X[3] = {x0, x1, x2};
#pragma unroll
  for (uint32_t Q = 1u << 9; Q > 1; Q >>= 1) {
    uint32_t P = Q - 1;
#pragma unroll
    for (int i = 0; i < 3; i++) {
      if (X[i] & Q) {
        X[0] ^= P;
      } else {
        uint32_t t = (X[0] ^ X[i]) & P;
        X[0] ^= t;
        X[i] ^= t;
      }
    }
  }
  X[1] ^= X[0];
  X[2] ^= X[1];
  uint32_t t = 0;
#pragma unroll
  for (uint32_t Q = 1u << 9; Q > 1; Q >>= 1)
    if (X[2] & Q) t ^= Q - 1;
  X[0] ^= t; X[1] ^= t; X[2] ^= t;
  uint32_t key = 0;
#pragma unroll
  for (int lev = 9; lev >= 0; lev--)
    key = (key << 3) | (((X[0] >> lev) & 1u) << 2) | (((X[1] >> lev) & 1u) << 1) |
          ((X[2] >> lev) & 1u);
  return key;
}

// Morton (Z-order) key of the same quantised cell: bits interleaved level by level, axis 0
// most significant within a level. Used only when a comparison run selects it.
__device__ __forceinline__ uint32_t morton30(uint32_t x0, uint32_t x1, uint32_t x2) {
  uint32_t key = 0;
#pragma unroll
  for (int lev = 9; lev >= 0; lev--)
    key = (key << 3) | (((x0 >> lev) & 1u) << 2) | (((x1 >> lev) & 1u) << 1) | ((x2 >> lev) & 1u);
  return key;
}

__global__ void k_wrap_key(int32_t n, int curve, double Lx, double Ly, double Lz,
                           const float* __restrict__ pos,
                           const int32_t* __restrict__ species, const float* __restrict__ vel,
                           const float* __restrict__ forces, const int32_t* __restrict__ pa,
                           float* __restrict__ pos_w, uint32_t* __restrict__ key,
                           int32_t* __restrict__ idx, int32_t* __restrict__ sp_tmp,
                           float* __restrict__ v_tmp, float* __restrict__ f_tmp,
                           int32_t* __restrict__ pa_tmp, int32_t* __restrict__ status,
                           int32_t* __restrict__ cell_start, int32_t* __restrict__ cell_fill,
                           int64_t ncell, int32_t* __restrict__ misc,
                           int32_t* __restrict__ row_end) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  // counters of the later stages start at zero: cell counts (ncell + 1, the last one for the
  // scan's total), cell fill counters, the row statistics and the last row offset
  const int64_t nclr = ncell + 1 > 16 ? ncell + 1 : 16;
  for (int64_t j = i; j < nclr; j += (int64_t)gridDim.x * blockDim.x) {
    if (j <= ncell) cell_start[j] = 0;
    if (j < ncell) cell_fill[j] = 0;
    if (j < 16) misc[j] = 0;
  }
  if (i == 0) *row_end = 0;
  if (i >= n) return;
  // a non-finite coordinate is reported through the status word (its key and cell are then
  // meaningless but stay in range: the quantisation and the cell index clamp)
  if (!(isfinite(pos[3 * i]) && isfinite(pos[3 * i + 1]) && isfinite(pos[3 * i + 2])))
    atomicOr(status, kStatusNonFinite);
  float x = wrap_coord(pos[3 * i + 0], Lx);
  float y = wrap_coord(pos[3 * i + 1], Ly);
  float z = wrap_coord(pos[3 * i + 2], Lz);
  pos_w[3 * i + 0] = x;
  pos_w[3 * i + 1] = y;
  pos_w[3 * i + 2] = z;
  const uint32_t q0 = quant10(x, Lx), q1 = quant10(y, Ly), q2 = quant10(z, Lz);
  key[i] = curve == 1 ? morton30(q0, q1, q2) : hilbert30(q0, q1, q2);
  idx[i] = i;
  sp_tmp[i] = species[i];
  if (vel)
    for (int a = 0; a < 3; a++) v_tmp[3 * i + a] = vel[3 * i + a];
  if (forces)
    for (int a = 0; a < 3; a++) f_tmp[3 * i + a] = forces[3 * i + a];
  if (pa) pa_tmp[i] = pa[i];
}

__global__ void __launch_bounds__(256) k_radix_hist(const uint32_t* __restrict__ keys, int32_t n,
                                                    int shift, int32_t* __restrict__ hist,
                                                    int32_t nblk) {
  __shared__ int32_t cnt[256];
  int t = threadIdx.x;
  cnt[t] = 0;
  __syncthreads();
  int64_t base = (int64_t)blockIdx.x * kTile;
  for (int r = 0; r < kTile / 256; r++) {
    int64_t i = base + r * 256 + t;
    if (i < n) atomicAdd(&cnt[(keys[i] >> shift) & 255u], 1);
  }
  __syncthreads();
  hist[(int64_t)t * nblk + blockIdx.x] = cnt[t];
}

// Stable scatter of one 8-bit digit. Items are visited in index order (round, wave, lane);
// within a wave the rank among equal digits comes from 8 ballots.
__global__ void __launch_bounds__(256) k_radix_scatter(const uint32_t* __restrict__ kin,
                                                       const int32_t* __restrict__ vin,
                                                       uint32_t* __restrict__ kout,
                                                       int32_t* __restrict__ vout, int32_t n,
                                                       int shift, const int32_t* __restrict__ hist,
                                                       int32_t nblk) {
  __shared__ int32_t base_off[256];
  __shared__ int32_t run[256];
  __shared__ int32_t wcnt[4][256];
  int t = threadIdx.x, w = t >> 6, lane = t & 63;
  base_off[t] = hist[(int64_t)t * nblk + blockIdx.x];
  run[t] = 0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int64_t base = (int64_t)blockIdx.x * kTile;
  for (int r = 0; r < kTile / 256; r++) {
#pragma unroll
    for (int ww = 0; ww < 4; ww++) wcnt[ww][t] = 0;
    __syncthreads();
    int64_t i = base + r * 256 + t;
    bool valid = i < n;
    uint32_t key = valid ? kin[i] : 0u;
    uint32_t d = (key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; b++) {
      bool bit = (d >> b) & 1u;
      uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    int rank = __popcll(peers & lt);
    if (valid && rank == 0) wcnt[w][d] = __popcll(peers);
    __syncthreads();
    {
      int acc = run[t];
#pragma unroll
      for (int ww = 0; ww < 4; ww++) {
        int c = wcnt[ww][t];
        wcnt[ww][t] = acc;
        acc += c;
      }
      run[t] = acc;
    }
    __syncthreads();
    if (valid) {
      int64_t p = (int64_t)base_off[d] + wcnt[w][d] + rank;
      kout[p] = key;
      vout[p] = vin[i];
    }
    __syncthreads();
  }
}

struct CellGrid {
  int nc[3];
  double L[3];
};

__device__ __forceinline__ int cell_coord(float x, int nc, double L) {
  int v = (int)floor((double)x * (double)nc / L);
  return v < 0 ? 0 : (v >= nc ? nc - 1 : v);
}

// atomicAdd(&cnt[c], 1) for every active lane, one atomic per distinct c in the wave; returns
// the lane's slot (the counter's old value plus the rank among the lanes with the same c,
// ranks in lane order)
__device__ __forceinline__ int32_t wave_aggregated_add(int32_t* __restrict__ cnt, int c) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t left = __ballot(1);
  int32_t slot = 0;
  while (left) {
    const int lead = __builtin_ctzll(left);
    const int cl = __builtin_amdgcn_readlane(c, lead);
    const uint64_t m = __ballot(c == cl) & left;
    int32_t b = 0;
    if (lane == lead) b = atomicAdd(&cnt[cl], __popcll(m));
    b = __builtin_amdgcn_readlane(b, lead);
    if (c == cl) slot = b + __popcll(m & lt);
    left &= ~m;
  }
  return slot;
}

__global__ void k_permute(int32_t n, const int32_t* __restrict__ idx, const uint32_t* __restrict__ key,
                          const float* __restrict__ pos_w, const int32_t* __restrict__ sp_tmp,
                          const float* __restrict__ v_tmp, const float* __restrict__ f_tmp,
                          const int32_t* __restrict__ pa_tmp, float* __restrict__ pos,
                          int32_t* __restrict__ species, float* __restrict__ vel,
                          float* __restrict__ forces, int32_t* __restrict__ pa,
                          float* __restrict__ ref_pos, int32_t* __restrict__ perm,
                          uint32_t* __restrict__ hkey, CellGrid g,
                          int32_t* __restrict__ cell_id, int32_t* __restrict__ cell_cnt) {
  int32_t k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  int32_t o = idx[k];
  float x = pos_w[3 * o], y = pos_w[3 * o + 1], z = pos_w[3 * o + 2];
  pos[3 * k] = x; pos[3 * k + 1] = y; pos[3 * k + 2] = z;
  // cell of the sorted atom, counted with one atomic per distinct cell of the wave
  // (consecutive atoms along the curve mostly share a cell)
  const int c = (cell_coord(x, g.nc[0], g.L[0]) * g.nc[1] + cell_coord(y, g.nc[1], g.L[1])) *
                    g.nc[2] + cell_coord(z, g.nc[2], g.L[2]);
  cell_id[k] = c;
  (void)wave_aggregated_add(cell_cnt, c);
  if (ref_pos) { ref_pos[3 * k] = x; ref_pos[3 * k + 1] = y; ref_pos[3 * k + 2] = z; }
  species[k] = sp_tmp[o];
  if (vel)
    for (int a = 0; a < 3; a++) vel[3 * k + a] = v_tmp[3 * o + a];
  if (forces)
    for (int a = 0; a < 3; a++) forces[3 * k + a] = f_tmp[3 * o + a];
  if (pa) pa[k] = pa_tmp[o];
  perm[k] = o;
  if (hkey) hkey[k] = key[k];
}

// Cell-sorted copy of the atoms: atoms[slot] = i and cpos[slot] = (x_i, y_i, z_i, bits of i),
// so a cell's atoms and their positions are contiguous (one 16-byte load per candidate).
__global__ void k_cell_fill(int32_t n, const int32_t* __restrict__ cell_id,
                            const int32_t* __restrict__ cell_start, int32_t* __restrict__ fill,
                            int32_t* __restrict__ atoms, const float* __restrict__ pos,
                            float4* __restrict__ cpos) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int c = cell_id[i];
  const int slot = cell_start[c] + wave_aggregated_add(fill, c);
  atoms[slot] = i;
  cpos[slot] = make_float4(pos[3 * i], pos[3 * i + 1], pos[3 * i + 2], __int_as_float(i));
}

// Stencil cell v (0..26) of cell c: the neighbour cell's index and the image-shift code
// 9(sx+1) + 3(sy+1) + (sz+1) of its wrap.
__device__ __forceinline__ void stencil_cell(int c, int v, const CellGrid& g, int& cell,
                                             int& code) {
  const int cz = c % g.nc[2], cy = (c / g.nc[2]) % g.nc[1], cx = c / (g.nc[1] * g.nc[2]);
  const int d[3] = {v / 9 - 1, (v / 3) % 3 - 1, v % 3 - 1};
  int cc[3] = {cx + d[0], cy + d[1], cz + d[2]};
  int sh[3];
  for (int a = 0; a < 3; a++) {
    sh[a] = 0;
    if (cc[a] < 0) { cc[a] += g.nc[a]; sh[a] = -1; }
    else if (cc[a] >= g.nc[a]) { cc[a] -= g.nc[a]; sh[a] = 1; }
  }
  cell = (cc[0] * g.nc[1] + cc[1]) * g.nc[2] + cc[2];
  code = 9 * (sh[0] + 1) + 3 * (sh[1] + 1) + (sh[2] + 1);
}

// The fp64 pair test (operation order fixed, contraction off): candidate at fp32 (x, y, z)
// with shift code `code` against atom i at (xi0, xi1, xi2).
__device__ __forceinline__ bool pair_pass(float x, float y, float z, int code, double xi0,
                                          double xi1, double xi2, const CellGrid& g,
                                          double rcs2) {
  const double s0 = (double)(code / 9 - 1), s1 = (double)((code / 3) % 3 - 1),
               s2 = (double)(code % 3 - 1);
  const double r0 = ((double)x - xi0) + s0 * g.L[0];
  const double r1 = ((double)y - xi1) + s1 * g.L[1];
  const double r2 = ((double)z - xi2) + s2 * g.L[2];
  double rr = r0 * r0 + r1 * r1;
  rr = rr + r2 * r2;
  return rr < rcs2;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Pair search of one atom by one wave with the candidates read from global memory
// (cell-sorted positions; stencil cells vstart/vcode/vpre in LDS), for cells whose stencil
// holds more candidates than the LDS stage. FILL = false returns the count; FILL = true
// writes the row sorted by (j, code) through the wave's LDS buffer `buf` (kMaxRow entries).
template <bool FILL>
__device__ int atom_row_global(int32_t i, int lane, const CellGrid& g, double rcs2,
                               const float4* __restrict__ cpos, const int32_t* vstart,
                               const int32_t* vcode, const int32_t* vpre,
                               const int32_t* __restrict__ row_ptr,
                               uint32_t* __restrict__ col_shift, uint32_t* buf,
                               const float* __restrict__ pos) {
  const double xi0 = (double)pos[3 * i], xi1 = (double)pos[3 * i + 1], xi2 = (double)pos[3 * i + 2];
  const int total = vpre[27];
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int count = 0;
  for (int q0 = 0; q0 < total; q0 += 64) {
    const int q = q0 + lane;
    const bool ok = q < total;
    int lo = 0, hi = 27;  // stencil cell v with vpre[v] <= q < vpre[v+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (vpre[mid] <= q) lo = mid; else hi = mid;
    }
    const float4 p = cpos[ok ? vstart[lo] + (q - vpre[lo]) : 0];
    const int32_t j = __float_as_int(p.w);
    const int code = vcode[lo];
    const bool pass = ok && pair_pass(p.x, p.y, p.z, code, xi0, xi1, xi2, g, rcs2) &&
                      !(j == i && code == 13);
    const uint64_t m = __ballot(pass);
    if (FILL) {
      const int slot = count + __popcll(m & lt);
      if (pass && slot < kMaxRow) buf[slot] = ((uint32_t)j << 5) | (uint32_t)code;
    }
    count += __popcll(m);
  }
  if (!FILL || count > kMaxRow) return count;  // long rows are rejected before the fill
  const int64_t o = row_ptr[i];
  wave_sync_lds();
  int p2 = 1;
  while (p2 < count) p2 <<= 1;
  for (int k = count + lane; k < p2; k += 64) buf[k] = 0xFFFFFFFFu;
  wave_sync_lds();
  for (int k = 2; k <= p2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int u = lane; u < (p2 >> 1); u += 64) {
        const int a = 2 * jj * (u / jj) + (u % jj);
        const int b = a + jj;
        const uint32_t va = buf[a], vb = buf[b];
        const bool up = (a & k) == 0;
        if ((va > vb) == up) { buf[a] = vb; buf[b] = va; }
      }
      wave_sync_lds();
    }
  }
  for (int k = lane; k < count; k += 64) {
    const uint32_t e = buf[k];
    col_shift[o + k] = (e >> 5) | ((e & 31u) << 27);
  }
  wave_sync_lds();
  return count;
}

// Candidates a cell block stages in LDS (16 bytes each). 2016 rather than 2048 keeps the
// block's LDS (with the stencil tables) within 32 KiB, so five blocks fit a CU.
constexpr int kCellCap = 2016;

// Image-shifted fp32 position of a candidate with shift code `code` (one rounding per axis);
// the staging and the sorted fill compute it the same way from the same stored coordinates.
__device__ __forceinline__ float3 shifted_pos(float x, float y, float z, int code,
                                              const CellGrid& g) {
  return make_float3(x + (float)(code / 9 - 1) * (float)g.L[0],
                     y + (float)((code / 3) % 3 - 1) * (float)g.L[1],
                     z + (float)(code % 3 - 1) * (float)g.L[2]);
}

// Sorts the block's staged candidates by their entry (j << 5 | shift code; distinct within a
// stencil) and leaves them in that order in spos[0, total), with their image-shifted
// positions. On entry, thread t holds candidate q = t + 256 r in sp[r] (r < kPer; the entry's
// bits in .w) and spos is free; total <= 256 * EPT. The 32-bit entries are sorted by an
// ascending bitonic network in registers: position a = t*EPT + r lives in thread t, so a
// compare-exchange at distance jj < EPT stays in the thread, one with EPT <= jj < 64*EPT
// crosses lanes of a wave (DPP moves, or a lane shuffle for lanes 16 and 32 apart), and only
// the three stages with partners in another wave exchange through LDS (spos as scratch).
// Each sorted entry then reads its atom's stored position again (pos[3j..3j+2], mostly an L2
// hit: the staging has just read it) and shifts it, so only the 4-byte entries travel
// through the network.
template <int J, int EPT>
__device__ __forceinline__ void bitonic_in_thread(uint32_t (&x)[EPT], int base, int k) {
#pragma unroll
  for (int r = 0; r < EPT; r++)
    if ((r & J) == 0) {
      const bool up = ((base + r) & k) == 0;
      const uint32_t a = x[r], b = x[r | J];
      const uint32_t lo = min(a, b), hi = max(a, b);
      x[r] = up ? lo : hi;
      x[r | J] = up ? hi : lo;
    }
}

// The value of lane (lane ^ m) for m a power of two below 64. Distances 1, 2, 4 and 8 stay
// in the VALU as DPP moves: quad permutations [1,0,3,2] and [2,3,0,1]; a half-row mirror
// (lane ^ 7) followed by the quad reversal (lane ^ 3) for 4; a rotation by 8 within a row of
// 16 lanes for 8. Distances 16 and 32 use ds_bpermute, which goes through the LDS unit.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, int m) {
  const int x = (int)v;
  switch (m) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
    case 4: {
      const int t = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, false);
    }
    case 8: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);
    default: return (uint32_t)__shfl_xor(x, m, 64);
  }
}

template <int EPT, int kPer>
__device__ __forceinline__ void sort_staged(float4* spos, const float4 (&sp)[kPer], int total,
                                            int t, const float* __restrict__ pos,
                                            const CellGrid& g) {
  static_assert(EPT <= kPer, "every key slot has a staged candidate slot");
  constexpr int N = 256 * EPT;
  const int base = t * EPT;
  uint32_t x[EPT];
#pragma unroll
  for (int r = 0; r < EPT; r++) {
    const int q = t + 256 * r;
    x[r] = q < total ? __float_as_uint(sp[r].w) : 0xFFFFFFFFu;  // above every entry
  }
  uint32_t* xbuf = reinterpret_cast<uint32_t*>(spos);  // N * 4 bytes <= spos
  // fully unrolled: every stage's distances are compile-time constants
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj >= 64 * EPT) {  // block-uniform
        __syncthreads();     // earlier readers of xbuf are done
#pragma unroll
        for (int r = 0; r < EPT; r++) xbuf[base + r] = x[r];
        __syncthreads();
#pragma unroll
        for (int r = 0; r < EPT; r++) {
          const int a = base + r;
          const uint32_t y = xbuf[a ^ jj];
          const bool keep_min = ((a & jj) == 0) == ((a & k) == 0);
          x[r] = keep_min ? min(x[r], y) : max(x[r], y);
        }
      } else if (jj >= EPT) {
        const int m = jj / EPT;  // lane distance (a power of two below 64)
#pragma unroll
        for (int r = 0; r < EPT; r++) {
          const int a = base + r;
          const uint32_t y = lane_xor_u32(x[r], m);
          const bool keep_min = ((a & jj) == 0) == ((a & k) == 0);
          x[r] = keep_min ? min(x[r], y) : max(x[r], y);
        }
      } else if (jj == 1) {
        bitonic_in_thread<1, EPT>(x, base, k);
      } else if (jj == 2) {
        bitonic_in_thread<2, EPT>(x, base, k);
      } else {
        if constexpr (EPT > 4) bitonic_in_thread<4, EPT>(x, base, k);
      }
    }
  }
  // positions of the sorted entries (requested together, then written once the last
  // exchange reads are done); positions in [total, kCellCap) take filler that the pair loop
  // never reads
  float4 v[EPT];
#pragma unroll
  for (int r = 0; r < EPT; r++) {
    const uint32_t e = base + r < total ? x[r] : 0u;
    const int32_t j = (int32_t)(e >> 5);
    v[r] = make_float4(pos[3 * j], pos[3 * j + 1], pos[3 * j + 2], __uint_as_float(e));
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < EPT; r++)
    if (base + r < kCellCap) {
      const float3 ps = shifted_pos(v[r].x, v[r].y, v[r].z, (int)(x[r] & 31u), g);
      spos[base + r] = make_float4(ps.x, ps.y, ps.z, v[r].w);
    }
}

// Pair search with LDS-staged cell stencils: one 256-thread block per cell (the second level
// of the three-level search). The block stages the candidates of the cell's 27-cell stencil
// (image-shifted fp32 position and entry j<<5|code, one 16-byte load each) in LDS once; the
// fill pass also sorts them by (j, code) with a bitonic sort, so the ballot compaction of each
// atom's passing candidates comes out in the row's order and is written to the CSR directly.
// The four waves take the cell's atoms in turn and test them against the staged candidates
// (the third level). The decision is the fp64 test of pair_pass; an fp32 distance decides
// first wherever it cannot differ from it: pairs whose fp32 squared distance lies more than
// `band` away from (r_cut+skin)^2 (band bounds the fp32 rounding of the shifted position, the
// difference and the squares, computed on the host) are classified by it, the few inside the
// band by the fp64 test from the stored positions. A stencil with more than kCellCap
// candidates (small or dense boxes) is read from global memory per atom instead (fp64 test).
// FILL = false writes each atom's count to row_ptr[i].
constexpr int kCellAtoms = 4;  // atoms a wave tests against each candidate it reads
template <bool FILL>
__global__ void __launch_bounds__(256) k_cell_pairs(CellGrid g, double rcs2, float lo2, float hi2,
                                                    const float* __restrict__ pos,
                                                    const float4* __restrict__ cpos,
                                                    const int32_t* __restrict__ cell_start,
                                                    const int32_t* __restrict__ cell_atoms,
                                                    int32_t* __restrict__ row_ptr,
                                                    uint32_t* __restrict__ col_shift) {
  __shared__ int32_t vstart[27], vcode[27], vpre[28];
  // staged candidates (float4; for the fill in (j, shift) order); the global-memory path
  // reuses the space as four per-wave row buffers
  constexpr int kBytes = kCellCap * 16;
  static_assert(kBytes >= 4 * kMaxRow * 4, "row buffers fit the staging area");
  __shared__ __align__(16) char smem[kBytes];
  float4* spos = reinterpret_cast<float4*>(smem);
  const int t = threadIdx.x, lane = t & 63;
  // the wave index, known to the compiler as wave-uniform (keeps the per-atom conditions and
  // counts scalar)
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c = (int)xcd_block(blockIdx.x, gridDim.x);
  // the cell's atom range, wave-uniform (scalar registers, scalar per-atom conditions)
  const int32_t a0 = __builtin_amdgcn_readfirstlane(cell_start[c]);
  const int32_t a1 = __builtin_amdgcn_readfirstlane(cell_start[c + 1]);
  if (a0 == a1) return;  // empty cell (the whole block returns)
  if (t < 64) {
    int32_t sz = 0;
    if (lane < 27) {
      int cell, code;
      stencil_cell(c, lane, g, cell, code);
      const int32_t s0 = cell_start[cell];
      vstart[lane] = s0;
      vcode[lane] = code;
      sz = cell_start[cell + 1] - s0;
    }
    int32_t inc = sz;  // inclusive prefix of the 27 sizes across lanes
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const int32_t y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane < 27) vpre[lane + 1] = inc;
    if (lane == 0) vpre[0] = 0;
  }
  __syncthreads();
  const int total = vpre[27];
  if (total > kCellCap) {  // uniform across the block
    uint32_t* buf = reinterpret_cast<uint32_t*>(smem) + wv * kMaxRow;
    for (int32_t k = a0 + wv; k < a1; k += 4) {
      const int32_t i = cell_atoms[k];
      const int cnt = atom_row_global<FILL>(i, lane, g, rcs2, cpos, vstart, vcode, vpre, row_ptr,
                                            col_shift, buf, pos);
      if (!FILL && lane == 0) row_ptr[i] = cnt;
    }
    return;
  }
  // stage candidate q of stencil cell v (vpre[v] <= q < vpre[v+1]). A thread's candidates
  // (at most kPer) first find their stencil cells, then request their positions
  // together.
  constexpr int kPer = (kCellCap + 255) / 256;
  int sv[kPer];
#pragma unroll
  for (int r = 0; r < kPer; r++) {
    const int q = t + 256 * r;
    int lo = 0, hi = 27;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (vpre[mid] <= q) lo = mid; else hi = mid;
    }
    sv[r] = lo;
  }
  float4 sp[kPer];
#pragma unroll
  for (int r = 0; r < kPer; r++) {
    const int q = t + 256 * r;
    sp[r] = q < total ? cpos[vstart[sv[r]] + (q - vpre[sv[r]])] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int r = 0; r < kPer; r++) {
    const int q = t + 256 * r;
    if (q < total) {
      const float4 p = sp[r];
      const int code = vcode[sv[r]];
      const uint32_t entry = ((uint32_t)__float_as_int(p.w) << 5) | (uint32_t)code;
      if (FILL) {  // the sort shifts the positions after sorting the entries
        sp[r].w = __uint_as_float(entry);
      } else {
        const float3 ps = shifted_pos(p.x, p.y, p.z, code, g);
        spos[q] = make_float4(ps.x, ps.y, ps.z, __uint_as_float(entry));
      }
    }
  }
  if (FILL) {  // the entries of one stencil are distinct; block-uniform choice
    if (total <= 1024) sort_staged<4>(spos, sp, total, t, pos, g);
    else sort_staged<8>(spos, sp, total, t, pos, g);
  }
  __syncthreads();
  // Each wave takes kCellAtoms of the cell's atoms at a time: every staged candidate read
  // from LDS is tested against all of them. An atom meets itself once among the staged
  // candidates (its own cell with shift code 13, at fp32 distance exactly 0, so always
  // near): the count pass subtracts it once per atom, the fill pass drops the lane whose
  // entry is the atom's own (i << 5 | 13).
  for (int32_t k0 = a0 + wv * kCellAtoms; k0 < a1; k0 += 4 * kCellAtoms) {
    int32_t ia[kCellAtoms];
    uint32_t eself[kCellAtoms];
    float xf[kCellAtoms][3];
    int count[kCellAtoms];
    int64_t o[kCellAtoms];
#pragma unroll
    for (int u = 0; u < kCellAtoms; u++) {
      // atoms past the cell's end repeat its first atom (wave-uniform; never written)
      const int32_t i = cell_atoms[k0 + u < a1 ? k0 + u : a0];
      ia[u] = i;
      eself[u] = ((uint32_t)i << 5) | 13u;
      xf[u][0] = pos[3 * i];
      xf[u][1] = pos[3 * i + 1];
      xf[u][2] = pos[3 * i + 2];
      count[u] = FILL ? 0 : -1;
      o[u] = FILL ? (int64_t)row_ptr[i] : 0;
    }
    // one batch of 64 staged candidates (p: this lane's); the next batch's candidate is read
    // by the caller before this one is tested
    auto batch = [&](int q0, const float4 p) {
      const int q = q0 + lane;
      const bool ok = q < total;
      const uint32_t entry = __float_as_uint(p.w);
      // the decisions as wave masks (one compare each): near in fp32, and within the rounding
      // band of (r_cut+skin)^2 (checked once per batch)
      const uint64_t m_ok = __ballot(ok);
      float d2v[kCellAtoms];
      uint64_t m_near[kCellAtoms];
      uint64_t m_band = 0;
#pragma unroll
      for (int u = 0; u < kCellAtoms; u++) {
        const float dx = p.x - xf[u][0], dy = p.y - xf[u][1], dz = p.z - xf[u][2];
        d2v[u] = __builtin_fmaf(dz, dz, __builtin_fmaf(dy, dy, dx * dx));
        m_near[u] = __ballot(d2v[u] < lo2);
        m_band |= __ballot(d2v[u] <= hi2) & ~m_near[u];
      }
      // inside the band the fp64 test decides; one branch per batch keeps its fp64 shift
      // terms (shared by the atoms) out of the common path
      if ((m_band & m_ok) != 0ull) {  // wave-uniform, rare
        const int32_t j = (int32_t)(entry >> 5);
        const int code = (int)(entry & 31u);
#pragma unroll
        for (int u = 0; u < kCellAtoms; u++) {
          if (k0 + u >= a1) break;  // wave-uniform
          bool in = false;
          if (ok && d2v[u] >= lo2 && d2v[u] <= hi2)
            in = pair_pass(pos[3 * j], pos[3 * j + 1], pos[3 * j + 2], code, (double)xf[u][0],
                           (double)xf[u][1], (double)xf[u][2], g, rcs2);
          m_near[u] |= __ballot(in);
        }
      }
#pragma unroll
      for (int u = 0; u < kCellAtoms; u++) {
        // atoms past the cell's end (repeats of its first atom) are never written or counted
        uint64_t m = k0 + u < a1 ? m_near[u] & m_ok : 0ull;
        if (FILL) {
          m &= ~__ballot(entry == eself[u]);
          if ((m >> lane) & 1ull) {
            const int slot = count[u] + (int)__builtin_amdgcn_mbcnt_hi(
                                            (uint32_t)(m >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (slot < kMaxRow)
              col_shift[o[u] + slot] = (entry >> 5) | ((entry & 31u) << 27);
          }
        }
        count[u] += __popcll(m);
      }
    };
    // batches in pairs, so the prefetched candidate alternates between two registers
    float4 pa = spos[lane < total ? lane : 0];
    for (int q0 = 0; q0 < total; q0 += 128) {
      const int qb = q0 + 64 + lane;
      const float4 pb = spos[qb < total ? qb : 0];  // (past the end: a filler, masked)
      batch(q0, pa);
      if (q0 + 64 < total) {  // wave-uniform
        const int qa = q0 + 128 + lane;
        pa = spos[qa < total ? qa : 0];
        batch(q0 + 64, pb);
      }
    }
    if (!FILL && lane == 0) {
#pragma unroll
      for (int u = 0; u < kCellAtoms; u++)  // (an atom at a non-finite position meets nothing)
        if (k0 + u < a1) row_ptr[ia[u]] = max(count[u], 0);
    }
  }
}

// rev[e] = slot of the reverse pair (j <- i, 26 - code) of entry e = (i <- j, code). Rows are
// sorted by (j, code) with distinct entries, and the pair test is symmetric, so the reverse
// entry is in row j. Each pair is searched once, from the row of its smaller index: for an
// entry with j >= i the lane searches row j for (i, 26 - code) and writes both directions.
// One wave takes kRevRows consecutive rows: their j >= i entries (index, key, j) are compacted
// into LDS first, so every lane runs two interleaved searches (independent load chains).
// The search reads runs of four consecutive entries (one 16-byte request each, always inside
// row j): three runs spread over the open range per round cut it about four-fold, so a row of
// ~130 entries takes two or three dependent rounds instead of the eight probes of a binary
// search. A key that a row lacks (impossible for a symmetric list) ends its search unwritten.
constexpr int kRevRows = 2;

__device__ __forceinline__ uint32_t rev_sort_key(uint32_t c) {
  return ((c & 0x7FFFFFFu) << 5) | (c >> 27);
}

// four consecutive col entries from a 4-byte-aligned address
__device__ __forceinline__ uint4 load_run4(const uint32_t* p) {
  uint4 v;
  __builtin_memcpy(&v, p, sizeof(v));
  return v;
}

__global__ void __launch_bounds__(256) k_rev(int32_t n, const int32_t* __restrict__ row_ptr,
                                             const uint32_t* __restrict__ col,
                                             int32_t* __restrict__ rev) {
  __shared__ int32_t se[4][128];
  __shared__ uint32_t sw[4][128];
  __shared__ int32_t sj[4][128];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // XCD-aware block order: each XCD walks one contiguous range of rows, whose target rows
  // (spatial neighbours, nearby in curve order) then share that XCD's L2
  const int32_t i0 = ((int32_t)xcd_block(blockIdx.x, gridDim.x) * 4 + wv) * kRevRows;
  if (i0 >= n) return;
  const int32_t i1 = min(i0 + kRevRows, n);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t b = row_ptr[i0], e_end = row_ptr[i1];
  int32_t i = i0;  // row of entry b + lane advances with the entries
  for (int32_t base = b; base < e_end;) {
    // compact up to 128 searching entries (j >= i) of [base, e_end) into LDS
    int cnt = 0;
    int32_t e = base;
    while (e < e_end && cnt <= 64) {
      const int32_t ee = e + lane;
      bool want = false;
      uint32_t key = 0;
      int32_t j = 0;
      if (ee < e_end) {
        int32_t r = i;
        while (row_ptr[r + 1] <= ee) r++;  // rows of the wave's range, ascending
        const uint32_t c = col[ee];
        j = (int32_t)(c & 0x7FFFFFFu);
        want = j >= r;
        key = ((uint32_t)r << 5) | (26u - (c >> 27));
      }
      const uint64_t m = __ballot(want);
      if (want) {
        const int slot = cnt + __popcll(m & lt);
        se[wv][slot] = ee;
        sw[wv][slot] = key;
        sj[wv][slot] = j;
      }
      cnt += __popcll(m);
      e += 64;
    }
    base = e;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // search state: the open range [lo, hi) of row [rs, re); found = slot, -1 searching,
    // -2 no search (or a key the row lacks)
    int32_t lo[2], hi[2], rs[2], re[2], ei[2], found[2];
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int k = lane + 64 * h;
      ei[h] = -1;
      found[h] = -2;
      w[h] = 0;
      lo[h] = hi[h] = rs[h] = re[h] = 0;
      if (k < cnt) {
        ei[h] = se[wv][k];
        w[h] = sw[wv][k];
        const int32_t j = sj[wv][k];
        rs[h] = lo[h] = row_ptr[j];
        re[h] = hi[h] = row_ptr[j + 1];
        found[h] = -1;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
      if (found[h] == -1 && re[h] - rs[h] < 4) {  // short row: read its entries one by one
        found[h] = -2;
        for (int32_t k = rs[h]; k < re[h]; k++)
          if (rev_sort_key(col[k]) == w[h]) found[h] = k;
      }
    while (found[0] == -1 || found[1] == -1) {
      uint4 run[2][3];
      int32_t c0[2][3];
#pragma unroll
      for (int h = 0; h < 2; h++) {
        if (found[h] != -1) continue;
        const int32_t len = hi[h] - lo[h];
#pragma unroll
        for (int m = 0; m < 3; m++) {
          // runs inside [lo, hi) while it is longer than 4, else one run covering it; every
          // run lies in [rs, re) (re - rs >= 4)
          int32_t c = len > 4 ? lo[h] + ((m + 1) * len) / 4 - 2 : min(lo[h], re[h] - 4);
          if (len > 4) c = max(lo[h], min(c, hi[h] - 4));
          c0[h][m] = c;
          run[h][m] = load_run4(col + c);
        }
      }
#pragma unroll
      for (int h = 0; h < 2; h++) {
        if (found[h] != -1) continue;
        int32_t nlo = lo[h], nhi = hi[h];
        int32_t f = -1;
        bool lacks = false;
#pragma unroll
        for (int m = 0; m < 3; m++) {
          const uint32_t k0 = rev_sort_key(run[h][m].x), k1 = rev_sort_key(run[h][m].y),
                         k2 = rev_sort_key(run[h][m].z), k3 = rev_sort_key(run[h][m].w);
          const int32_t c = c0[h][m];
          if (w[h] < k0) nhi = min(nhi, c);
          else if (w[h] > k3) nlo = max(nlo, c + 4);
          else if (w[h] == k0) f = c;
          else if (w[h] == k1) f = c + 1;
          else if (w[h] == k2) f = c + 2;
          else if (w[h] == k3) f = c + 3;
          else lacks = true;
        }
        if (f >= 0) found[h] = f;
        else if (lacks || nlo >= nhi || hi[h] - lo[h] <= 4) found[h] = -2;
        lo[h] = nlo;
        hi[h] = nhi;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
      if (found[h] >= 0) {
        rev[ei[h]] = found[h];
        rev[found[h]] = ei[h];
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // the row of the next entries
    while (i < i1 - 1 && row_ptr[i + 1] <= base) i++;
  }
}

// Reverse index by row groups, for boxes at least 2 (r_cut + skin) wide on every axis: there a
// row holds at most one image of any atom, so its entries have distinct indices. A block takes
// kRevGroup consecutive rows [g, g + R). Their reverse entries in a target row j are the
// entries of row j with index in [g, g + R), which are consecutive there: for an entry
// e = (i <- j), rev[e] = lower_bound(row j, g) + #{rows i' in [g, i) that hold j}. So each
// distinct target row is searched once per group (about one search per eight entries for
// groups of 32 rows at water density), and every store rev[e] is contiguous. An LDS hash table
// maps each distinct target j to its search result and a mask of the group's rows holding it
// (OR-ed in any order, so the result does not depend on thread order). The group's entries
// (target and row) are first staged in LDS with independent loads, so neither pass over them
// waits on global memory. A group with more entries than the stage holds is split, and one
// whose table gets crowded (a probe chain of kRevMaxProbe) is redone in halves; a single row
// (at most kMaxRow = kRevSlots entries) always fits.
constexpr int kRevGroup = 32;
constexpr int kRevSlots = 1024;
constexpr int kRevMaxProbe = 64;   // probe chain that marks a group's table as crowded
constexpr int kRevEntries = 4608;  // entries of a group staged in LDS (32 rows of ~144)
static_assert(kRevEntries >= kMaxRow, "one row always fits the stage");
static_assert(kRevSlots >= kMaxRow, "one row's distinct targets always fit the table");
constexpr uint32_t kRevEmpty = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t rev_hash(uint32_t j) {
  return (j * 0x9E3779B1u) >> (32 - 10);  // kRevSlots = 2^10
}

// first position p in [rs, re] of the sorted row whose sort key is >= w, reading one run of
// four entries per round (the middle of the open range, or one run covering it once it is at
// most four long); NS independent searches advance in lockstep (act = false: none). One run
// per round keeps the number of memory instructions low (each costs the data-return path
// about the same whatever it carries), at the price of a few more rounds.
template <int NS>
__device__ __forceinline__ void lower_bound_runs(const uint32_t* __restrict__ col,
                                                 const bool (&act)[NS], const int32_t (&rs)[NS],
                                                 const int32_t (&re)[NS], uint32_t w,
                                                 int32_t (&out)[NS]) {
  int32_t lo[NS], hi[NS];
  bool live[NS];
#pragma unroll
  for (int h = 0; h < NS; h++) {
    lo[h] = rs[h];
    hi[h] = re[h];
    out[h] = rs[h];
    live[h] = act[h] && rs[h] < re[h];
    if (live[h] && re[h] - rs[h] < 4) {  // short row: count its entries below w
      int32_t p = rs[h];
      for (int32_t k = rs[h]; k < re[h]; k++)
        if (rev_sort_key(col[k]) < w) p = k + 1;
      out[h] = p;
      live[h] = false;
    }
  }
  for (;;) {
    bool any = false;
#pragma unroll
    for (int h = 0; h < NS; h++) any |= live[h];
    if (!any) break;
    uint4 run[NS];
    int32_t c0[NS];
#pragma unroll
    for (int h = 0; h < NS; h++) {
      if (!live[h]) continue;
      const int32_t len = hi[h] - lo[h];
      // inside [lo, hi) while it is longer than 4, else covering it; always inside [rs, re)
      // (re - rs >= 4)
      c0[h] = len > 4 ? lo[h] + (len - 4) / 2 : min(lo[h], re[h] - 4);
      run[h] = load_run4(col + c0[h]);
    }
#pragma unroll
    for (int h = 0; h < NS; h++) {
      if (!live[h]) continue;
      const bool covering = hi[h] - lo[h] <= 4;
      const int32_t q = (rev_sort_key(run[h].x) < w) + (rev_sort_key(run[h].y) < w) +
                        (rev_sort_key(run[h].z) < w) + (rev_sort_key(run[h].w) < w);
      const int32_t c = c0[h];
      // q > 0: every key before c + q is below w; q < 4: the key at c + q is not
      if (q > 0) lo[h] = max(lo[h], c + q);
      if (q < 4) hi[h] = min(hi[h], c + q);
      // a covering run pins the answer; otherwise the range shrank strictly
      if (covering || lo[h] >= hi[h]) {
        out[h] = lo[h];
        live[h] = false;
      }
    }
  }
}

__global__ void __launch_bounds__(256) k_rev_grouped(int32_t n,
                                                     const int32_t* __restrict__ row_ptr,
                                                     const uint32_t* __restrict__ col,
                                                     int32_t* __restrict__ rev) {
  __shared__ uint32_t tkey[kRevSlots];
  // per slot: (search result, mask of the group rows holding the target), read together
  __shared__ int2 tbm[kRevSlots];
  // the group's targets j in entry order; after the table pass, each entry's table slot and
  // group row (slot | row << 16), so the last pass reads them without probing the table
  __shared__ __align__(16) uint32_t sc[kRevEntries];
  __shared__ __align__(16) uint8_t srow[kRevEntries];  // their rows, offsets from the first
  __shared__ int16_t slist[kRevSlots];                 // occupied table slots
  __shared__ int32_t srp[kRevGroup + 1];
  __shared__ int32_t swsum[4];
  __shared__ int32_t sflag;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // XCD-aware block order: consecutive groups (spatial neighbours) share an XCD's L2
  const int32_t g0 = (int32_t)xcd_block(blockIdx.x, gridDim.x) * kRevGroup;
  if (g0 >= n) return;
  const int32_t g1 = min(g0 + kRevGroup, n);
  if (t <= g1 - g0) srp[t] = row_ptr[g0 + t];
  __syncthreads();
  int rcap = kRevGroup;
  int32_t ga = g0;
  while (ga < g1) {
    const int ra = (int)(ga - g0);
    int R = min(rcap, (int)(g1 - ga));
    while (R > 1 && srp[ra + R] - srp[ra] > kRevEntries) R >>= 1;  // block-uniform
    const int32_t e0 = srp[ra];
    const int ne = (int)(srp[ra + R] - e0);  // <= kRevEntries (one row: <= kMaxRow)
    // stage the group's targets, four consecutive entries per thread and load, and their rows;
    // clear the table
    for (int k = 4 * t; k < ne; k += 4 * 256) {
      uint4 v;
      if (k + 4 <= ne) {
        v = load_run4(col + e0 + k);
      } else {
        v.x = col[e0 + k];
        v.y = k + 1 < ne ? col[e0 + k + 1] : 0u;
        v.z = k + 2 < ne ? col[e0 + k + 2] : 0u;
        v.w = 0u;
      }
      const uint32_t m = 0x7FFFFFFu;
      *reinterpret_cast<uint4*>(&sc[k]) = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
    }
    for (int r = 0; r < R; r++)
      for (int k = (int)(srp[ra + r] - e0) + t; k < (int)(srp[ra + r + 1] - e0); k += 256)
        srow[k] = (uint8_t)r;
    for (int k = t; k < kRevSlots; k += 256) {
      tkey[k] = kRevEmpty;
      tbm[k].y = 0;
    }
    if (t == 0) sflag = 0;
    __syncthreads();
    // 1. distinct targets and the group rows holding each
    for (int k = t; k < ne; k += 256) {
      const uint32_t j = sc[k];
      uint32_t h = rev_hash(j);
      bool placed = false;
      // a group of several rows gives up on a long probe chain (a crowded table); a single
      // row may probe the whole table, where it always fits
      const int max_probe = R > 1 ? kRevMaxProbe : kRevSlots;
      for (int probe = 0; probe < max_probe; probe++) {
        const uint32_t old = atomicCAS(&tkey[h], kRevEmpty, j);
        if (old == kRevEmpty || old == j) {
          placed = true;
          break;
        }
        h = (h + 1) & (kRevSlots - 1);
      }
      if (!placed) {
        sflag = 1;
        break;
      }
      const uint32_t r = srow[k];
      atomicOr(reinterpret_cast<uint32_t*>(&tbm[h].y), 1u << r);
      sc[k] = h | (r << 16);  // the entry's slot and row (its target is no longer needed)
    }
    __syncthreads();
    const bool over = sflag != 0;
    if (over) {  // block-uniform: redo the group in halves
      rcap = R > 1 ? R / 2 : 1;
      __syncthreads();  // every thread has read sflag before the next attempt resets it
      continue;
    }
    // 2. list the occupied slots (thread t holds slots 4t .. 4t+3), then one search per
    //    distinct target: where its entries of index >= ga begin
    {
      uint32_t occ = 0;
#pragma unroll
      for (int u = 0; u < 4; u++) occ |= (tkey[4 * t + u] != kRevEmpty ? 1u : 0u) << u;
      int cnt = __popc(occ), inc = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      if (lane == 63) swsum[wv] = inc;
      __syncthreads();
      int off = inc - cnt;
      for (int k = 0; k < wv; k++) off += swsum[k];
#pragma unroll
      for (int u = 0; u < 4; u++)
        if (occ & (1u << u)) slist[off++] = (int16_t)(4 * t + u);
    }
    __syncthreads();
    const int nd = swsum[0] + swsum[1] + swsum[2] + swsum[3];
    for (int b0 = 0; b0 < nd; b0 += 2 * 256) {
      bool act[2];
      int32_t rs[2], re[2], out[2], slot[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; s2++) {
        const int k = b0 + 256 * s2 + t;
        act[s2] = k < nd;
        slot[s2] = act[s2] ? slist[k] : 0;
        rs[s2] = re[s2] = 0;
        if (act[s2]) {
          int2 b;
          __builtin_memcpy(&b, row_ptr + tkey[slot[s2]], sizeof(b));  // row_ptr[j], [j+1]
          rs[s2] = b.x;
          re[s2] = b.y;
        }
      }
      lower_bound_runs<2>(col, act, rs, re, (uint32_t)ga << 5, out);
#pragma unroll
      for (int s2 = 0; s2 < 2; s2++)
        if (act[s2]) tbm[slot[s2]].x = out[s2];
    }
    __syncthreads();
    // 3. every entry's reverse slot, four consecutive entries per thread and store
    for (int k = 4 * t; k < ne; k += 4 * 256) {
      const uint4 i4 = *reinterpret_cast<const uint4*>(&sc[k]);  // slot | row << 16
      const uint32_t info[4] = {i4.x, i4.y, i4.z, i4.w};
      int32_t v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        v[u] = 0;
        if (k + u < ne) {
          const uint32_t h = info[u] & 0xFFFFu;
          const uint32_t below = (1u << (info[u] >> 16)) - 1u;
          const int2 bm = tbm[h];
          v[u] = bm.x + __popc((uint32_t)bm.y & below);
        }
      }
      if (k + 4 <= ne) {
        const int4 o = make_int4(v[0], v[1], v[2], v[3]);
        __builtin_memcpy(rev + e0 + k, &o, sizeof(o));
      } else {
        for (int u = 0; u < 4 && k + u < ne; u++) rev[e0 + k + u] = v[u];
      }
    }
    __syncthreads();
    ga += R;
  }
}

// ---- scan -----------------------------------------------------------------------------
// Exclusive scan of int32 counts in place. Up to kScanOneMax entries one block of 1024
// threads does it in one launch (16 entries per thread); longer arrays take two launches
// (tile sums, then each tile adds the sum of the tile sums before it, which it reduces
// itself), and beyond kScanCarryTiles tiles a third launch scans the tile sums. Optionally
// the same launches report the largest count and the 64-bit total of the counts (stats[0],
// stats[2..3]) and copy one more word next to them (stats[1]), so that a caller reads all
// three with one copy.
constexpr int kScanTile = 4096;          // 256 threads x 16 (multi-block tiles)
constexpr int kScanOneMax = 16384;       // 1024 threads x 16
constexpr int kScanCarryTiles = 4096;

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int32_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

template <int NW>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* sh, int32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int32_t inc = wave_inclusive_scan(v);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  int32_t off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < NW; k++) {
    const int32_t x = sh[k];
    off += k < w ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// Largest value and 64-bit sum over the block, written by thread 0 (`atomic`: combined with
// what other blocks wrote; the targets then start at zero).
template <int NW>
__device__ __forceinline__ void block_stats(int32_t mx, unsigned long long sm, int32_t* stats,
                                            bool atomic) {
  __shared__ int32_t smx[NW];
  __shared__ unsigned long long ssm[NW];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o, 64));
    sm += __shfl_xor(sm, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    smx[threadIdx.x >> 6] = mx;
    ssm[threadIdx.x >> 6] = sm;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    mx = smx[0];
    sm = ssm[0];
    for (int k = 1; k < NW; k++) {
      mx = max(mx, smx[k]);
      sm += ssm[k];
    }
    unsigned long long* tot = reinterpret_cast<unsigned long long*>(stats + 2);
    if (atomic) {
      atomicMax(stats, mx);
      atomicAdd(tot, sm);
    } else {
      stats[0] = mx;
      *tot = sm;
    }
  }
}

// 16 consecutive entries from p (entries at or beyond n read as 0); 16-byte loads where the
// address allows
__device__ __forceinline__ void load16(const int32_t* __restrict__ d, int64_t base, int64_t n,
                                       int32_t v[16]) {
  if (base + 16 <= n && ((reinterpret_cast<uintptr_t>(d + base) & 15) == 0)) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int4 x = *reinterpret_cast<const int4*>(d + base + 4 * q);
      v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; k++) v[k] = (base + k < n) ? d[base + k] : 0;
  }
}

__device__ __forceinline__ void store16(int32_t* __restrict__ d, int64_t base, int64_t n,
                                        const int32_t v[16]) {
  if (base + 16 <= n && ((reinterpret_cast<uintptr_t>(d + base) & 15) == 0)) {
#pragma unroll
    for (int q = 0; q < 4; q++)
      *reinterpret_cast<int4*>(d + base + 4 * q) =
          make_int4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  } else {
#pragma unroll
    for (int k = 0; k < 16; k++)
      if (base + k < n) d[base + k] = v[k];
  }
}

__global__ void __launch_bounds__(1024) k_scan_one(int32_t* __restrict__ d, int32_t n,
                                                   int32_t* __restrict__ stats,
                                                   const int32_t* __restrict__ extra) {
  __shared__ int32_t sh[16];
  int32_t v[16];
  load16(d, threadIdx.x * 16, n, v);
  int32_t s = 0, mx = 0;
  unsigned long long sm = 0;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    s += v[k];
    mx = max(mx, v[k]);
    sm += (unsigned long long)(uint32_t)v[k];
  }
  int32_t tot;
  int32_t run = block_exclusive_scan<16>(s, sh, &tot);
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const int32_t y = v[k];
    v[k] = run;
    run += y;
  }
  store16(d, threadIdx.x * 16, n, v);
  if (stats) {
    block_stats<16>(mx, sm, stats, false);
    if (extra && threadIdx.x == 0) stats[1] = *extra;
  }
}

__global__ void __launch_bounds__(256) k_scan_partial(const int32_t* __restrict__ d, int64_t n,
                                                      int32_t* __restrict__ sums,
                                                      int32_t* __restrict__ stats,
                                                      const int32_t* __restrict__ extra) {
  int32_t v[16];
  load16(d, (int64_t)blockIdx.x * kScanTile + threadIdx.x * 16, n, v);
  int32_t s = 0, mx = 0;
  unsigned long long sm = 0;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    s += v[k];
    mx = max(mx, v[k]);
    sm += (unsigned long long)(uint32_t)v[k];
  }
  // block sum (wrapping in 32 bits like the scan itself)
  s = wave_inclusive_scan(s);
  __shared__ int32_t sh[4];
  if ((threadIdx.x & 63) == 63) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) sums[blockIdx.x] = sh[0] + sh[1] + sh[2] + sh[3];
  if (stats) {
    block_stats<4>(mx, sm, stats, true);
    if (extra && blockIdx.x == 0 && threadIdx.x == 0) stats[1] = *extra;
  }
}

__global__ void __launch_bounds__(256) k_scan_sums(int32_t* __restrict__ sums, int32_t nb) {
  __shared__ int32_t sh[4];
  int32_t carry = 0;
  for (int32_t b0 = 0; b0 < nb; b0 += 256) {
    int32_t k = b0 + threadIdx.x;
    int32_t v = k < nb ? sums[k] : 0;
    int32_t tot;
    int32_t ex = block_exclusive_scan<4>(v, sh, &tot);
    if (k < nb) sums[k] = carry + ex;
    carry += tot;
  }
}

// CARRY: the tile's offset is the sum of the tile sums before it (reduced here); otherwise
// `sums` already holds the scanned tile sums.
template <bool CARRY>
__global__ void __launch_bounds__(256) k_scan_final(int32_t* __restrict__ d, int64_t n,
                                                    const int32_t* __restrict__ sums) {
  __shared__ int32_t sh[4];
  int32_t carry;
  if (CARRY) {
    int32_t c = 0;
    for (int32_t b = threadIdx.x; b < (int32_t)blockIdx.x; b += 256) c += sums[b];
    int32_t tot;
    (void)block_exclusive_scan<4>(c, sh, &tot);
    carry = tot;
  } else {
    carry = sums[blockIdx.x];
  }
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * 16;
  int32_t v[16];
  load16(d, base, n, v);
  int32_t s = 0;
#pragma unroll
  for (int k = 0; k < 16; k++) s += v[k];
  int32_t tot;
  int32_t run = block_exclusive_scan<4>(s, sh, &tot) + carry;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const int32_t x = v[k];
    v[k] = run;
    run += x;
  }
  store16(d, base, n, v);
}

inline int32_t grid(int64_t n, int b) { return (int32_t)((n + b - 1) / b); }

}  // namespace

hipError_t scan_exclusive_i32(int32_t* data, int64_t n, int32_t* partial, hipStream_t s,
                              int32_t* stats, const int32_t* extra) {
  if (n <= 0) return hipSuccess;
  if (n <= kScanOneMax) {
    k_scan_one<<<1, 1024, 0, s>>>(data, (int32_t)n, stats, extra);
    return hipGetLastError();
  }
  const int64_t nb = (n + kScanTile - 1) / kScanTile;
  k_scan_partial<<<(unsigned)nb, 256, 0, s>>>(data, n, partial, stats, extra);
  if (nb <= kScanCarryTiles) {
    k_scan_final<true><<<(unsigned)nb, 256, 0, s>>>(data, n, partial);
  } else {
    k_scan_sums<<<1, 256, 0, s>>>(partial, (int32_t)nb);
    k_scan_final<false><<<(unsigned)nb, 256, 0, s>>>(data, n, partial);
  }
  return hipGetLastError();
}

hipError_t rev_index(int32_t n, const int32_t* row_ptr, const uint32_t* col, int32_t* rev,
                     hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_rev<<<grid(n, 4 * kRevRows), 256, 0, s>>>(n, row_ptr, col, rev);
  return hipGetLastError();
}

NbrWS carve_nbr(Carver& c, int32_t n) {
  NbrWS w{};
  int64_t nn = n > 0 ? n : 1;
  int64_t nblk = (nn + kTile - 1) / kTile;
  w.ncell_cap = 2 * nn + 64;
  w.pos_w = c.take<float>(3 * nn);
  w.key[0] = c.take<uint32_t>(nn);
  w.key[1] = c.take<uint32_t>(nn);
  w.idx[0] = c.take<int32_t>(nn);
  w.idx[1] = c.take<int32_t>(nn);
  w.hist = c.take<int32_t>(256 * nblk + 1);
  w.sp_tmp = c.take<int32_t>(nn);
  w.pa_tmp = c.take<int32_t>(nn);
  w.v_tmp = c.take<float>(3 * nn);
  w.f_tmp = c.take<float>(3 * nn);
  w.cell_start = c.take<int32_t>(w.ncell_cap + 1);
  w.cell_fill = c.take<int32_t>(w.ncell_cap);
  w.cell_atoms = c.take<int32_t>(nn);
  w.cell_pos = c.take<float4>(nn);
  w.cell_id = c.take<int32_t>(nn);
  int64_t scan_len = (256 * nblk + 1 > w.ncell_cap + 1 ? 256 * nblk + 1 : w.ncell_cap + 1);
  if (nn + 1 > scan_len) scan_len = nn + 1;
  w.scan_tmp = c.take<int32_t>(scan_len / kScanTile + 2);
  w.misc = c.take<int32_t>(16);
  return w;
}

int32_t build_neighbors_impl(int32_t n, const float box[3], float r_cut, float skin, float* pos,
                             int32_t* species, float* vel, float* ref_pos, float* forces,
                             int32_t* perm_accum, int32_t* perm, uint32_t* hkey,
                             int32_t* row_ptr, uint32_t* col_shift, int32_t* rev,
                             int64_t edge_cap, int64_t* n_edges, const NbrWS& ws,
                             int32_t* status, hipStream_t st) {
  const double L[3] = {(double)box[0], (double)box[1], (double)box[2]};
  const double rcs = (double)r_cut + (double)skin;
  const double rcs2 = rcs * rcs;
  // cell grid: cells at least (r_cut+skin)(1+1e-6) wide, at most ncell_cap of them
  CellGrid g;
  int64_t ncell = 1;
  for (int a = 0; a < 3; a++) {
    g.L[a] = L[a];
    int k = (int)floor(L[a] / (rcs * (1.0 + 1e-6)));
    g.nc[a] = k < 1 ? 1 : k;
  }
  for (;;) {
    ncell = (int64_t)g.nc[0] * g.nc[1] * g.nc[2];
    if (ncell <= ws.ncell_cap) break;
    int a = (g.nc[0] >= g.nc[1] && g.nc[0] >= g.nc[2]) ? 0 : (g.nc[1] >= g.nc[2] ? 1 : 2);
    g.nc[a]--;
  }
  // 1. wrap + keys (and the counters of the later stages cleared)
  k_wrap_key<<<grid(n, 256), 256, 0, st>>>(n, sort_curve(), L[0], L[1], L[2], pos, species,
                                           vel, forces,
                                           perm_accum, ws.pos_w, ws.key[0], ws.idx[0], ws.sp_tmp,
                                           ws.v_tmp, ws.f_tmp, ws.pa_tmp, status, ws.cell_start,
                                           ws.cell_fill, ncell, ws.misc, row_ptr + n);
  TESS_HIP_CHECK(hipGetLastError());
  // 2. stable radix sort, 4 x 8 bits (keys have 30 bits)
  int32_t nblk = grid(n, kTile);
  int cur = 0;
  for (int pass = 0; pass < 4; pass++) {
    int shift = 8 * pass;
    k_radix_hist<<<nblk, 256, 0, st>>>(ws.key[cur], n, shift, ws.hist, nblk);
    TESS_HIP_CHECK(scan_exclusive_i32(ws.hist, (int64_t)256 * nblk, ws.scan_tmp, st));
    TESS_TIMED("radix_scatter", st,
               k_radix_scatter<<<nblk, 256, 0, st>>>(ws.key[cur], ws.idx[cur], ws.key[cur ^ 1],
                                                     ws.idx[cur ^ 1], n, shift, ws.hist, nblk));
    TESS_HIP_CHECK(hipGetLastError());
    cur ^= 1;
  }
  // permute every per-atom array into sorted order, and count the atoms of each cell
  k_permute<<<grid(n, 256), 256, 0, st>>>(n, ws.idx[cur], ws.key[cur], ws.pos_w, ws.sp_tmp,
                                          vel ? ws.v_tmp : nullptr, forces ? ws.f_tmp : nullptr,
                                          perm_accum ? ws.pa_tmp : nullptr, pos, species, vel,
                                          forces, perm_accum, ref_pos, perm, hkey, g, ws.cell_id,
                                          ws.cell_start);
  TESS_HIP_CHECK(hipGetLastError());
  // 3. cells
  TESS_HIP_CHECK(scan_exclusive_i32(ws.cell_start, ncell + 1, ws.scan_tmp, st));
  k_cell_fill<<<grid(n, 256), 256, 0, st>>>(n, ws.cell_id, ws.cell_start, ws.cell_fill,
                                            ws.cell_atoms, pos, ws.cell_pos);
  TESS_HIP_CHECK(hipGetLastError());
  // 4. pairs: count, scan, check, fill
  // fp32 pre-decision band around (r_cut+skin)^2: bounds the fp32 error of the shifted
  // position (|x + sL| <= 2L), the difference and the fused squares for |d| <= r_cut+skin+2,
  // with a factor 16 to spare (u = 2^-24)
  const double Lmax = fmax(L[0], fmax(L[1], L[2]));
  const double band = 16.0 * ldexp(1.0, -24) * (2.0 * Lmax + rcs + 2.0) * (rcs + 2.0);
  const float lo2 = (float)(rcs2 - band), hi2 = (float)(rcs2 + band);
  TESS_TIMED("nbr_count", st,
             k_cell_pairs<false><<<(unsigned)ncell, 256, 0, st>>>(
                 g, rcs2, lo2, hi2, pos, ws.cell_pos, ws.cell_start, ws.cell_atoms, row_ptr,
                 nullptr));
  TESS_HIP_CHECK(hipGetLastError());
  // the scan also writes the longest row (misc[0]), a copy of the status word (misc[1]) and
  // the 64-bit pair total (misc[2..3]), read back with one copy: it adds in 32 bits, so a total
  // beyond the int32 range of row_ptr wraps there, while each row's count is still the
  // difference of its (wrapped) bounds and the 64-bit sum is exact
  TESS_HIP_CHECK(scan_exclusive_i32(row_ptr, (int64_t)n + 1, ws.scan_tmp, st, ws.misc, status));
  int32_t rb[4] = {0, 0, 0, 0};
  TESS_HIP_CHECK(hipMemcpyAsync(rb, ws.misc, sizeof(rb), hipMemcpyDeviceToHost, st));
  TESS_HIP_CHECK(hipStreamSynchronize(st));
  const int32_t max_row = rb[0], bits = rb[1];
  unsigned long long pairs = 0;
  std::memcpy(&pairs, rb + 2, sizeof(pairs));
  *n_edges = (int64_t)pairs;
  if (bits) {  // reported here and cleared (a pending bit may come from an earlier pass)
    TESS_HIP_CHECK(hipMemsetAsync(status, 0, sizeof(int32_t), st));
    return status_error(bits);
  }
  if (max_row > kMaxRow) return TESS_ERR_ROW;
  // a total that row_ptr (int32) cannot hold is reported like a capacity shortfall, with the
  // true count; no edge_cap satisfies it
  if ((int64_t)pairs > edge_cap || pairs > (unsigned long long)INT32_MAX) return TESS_ERR_CAPACITY;
  TESS_TIMED("nbr_fill", st,
             k_cell_pairs<true><<<(unsigned)ncell, 256, 0, st>>>(
                 g, rcs2, lo2, hi2, pos, ws.cell_pos, ws.cell_start, ws.cell_atoms, row_ptr,
                 col_shift));
  TESS_HIP_CHECK(hipGetLastError());
  if (rev) {
    // row groups need distinct indices per row: every box edge at least 2 (r_cut + skin)
    if (fmin(L[0], fmin(L[1], L[2])) >= 2.0 * rcs * (1.0 + 1e-6))
      k_rev_grouped<<<grid(n, kRevGroup), 256, 0, st>>>(n, row_ptr, col_shift, rev);
    else
      k_rev<<<grid(n, 4 * kRevRows), 256, 0, st>>>(n, row_ptr, col_shift, rev);
    TESS_HIP_CHECK(hipGetLastError());
  }
  return TESS_OK;
}

}  // namespace tess
