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
                           int32_t* __restrict__ pa_tmp, int32_t* __restrict__ status) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
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

__global__ void k_permute(int32_t n, const int32_t* __restrict__ idx, const uint32_t* __restrict__ key,
                          const float* __restrict__ pos_w, const int32_t* __restrict__ sp_tmp,
                          const float* __restrict__ v_tmp, const float* __restrict__ f_tmp,
                          const int32_t* __restrict__ pa_tmp, float* __restrict__ pos,
                          int32_t* __restrict__ species, float* __restrict__ vel,
                          float* __restrict__ forces, int32_t* __restrict__ pa,
                          float* __restrict__ ref_pos, int32_t* __restrict__ perm,
                          uint32_t* __restrict__ hkey) {
  int32_t k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  int32_t o = idx[k];
  float x = pos_w[3 * o], y = pos_w[3 * o + 1], z = pos_w[3 * o + 2];
  pos[3 * k] = x; pos[3 * k + 1] = y; pos[3 * k + 2] = z;
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

struct CellGrid {
  int nc[3];
  double L[3];
};

__device__ __forceinline__ int cell_coord(float x, int nc, double L) {
  int v = (int)floor((double)x * (double)nc / L);
  return v < 0 ? 0 : (v >= nc ? nc - 1 : v);
}

__global__ void k_cell_count(int32_t n, CellGrid g, const float* __restrict__ pos,
                             int32_t* __restrict__ cell_id, int32_t* __restrict__ cnt) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int cx = cell_coord(pos[3 * i], g.nc[0], g.L[0]);
  int cy = cell_coord(pos[3 * i + 1], g.nc[1], g.L[1]);
  int cz = cell_coord(pos[3 * i + 2], g.nc[2], g.L[2]);
  int c = (cx * g.nc[1] + cy) * g.nc[2] + cz;
  cell_id[i] = c;
  atomicAdd(&cnt[c], 1);
}

// Cell-sorted copy of the atoms: atoms[slot] = i and cpos[slot] = (x_i, y_i, z_i, bits of i),
// so a cell's atoms and their positions are contiguous (one 16-byte load per candidate).
__global__ void k_cell_fill(int32_t n, const int32_t* __restrict__ cell_id,
                            const int32_t* __restrict__ cell_start, int32_t* __restrict__ fill,
                            int32_t* __restrict__ atoms, const float* __restrict__ pos,
                            float4* __restrict__ cpos) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int c = cell_id[i];
  int slot = cell_start[c] + atomicAdd(&fill[c], 1);
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
constexpr int kCellCap = 2048;
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
  // staged candidates (float4) and, for the fill, the sort keys (entry << 32 | index); the
  // global-memory path reuses the space as four per-wave row buffers
  constexpr int kBytes = kCellCap * 16 + (FILL ? kCellCap * 8 : 0);
  static_assert(kBytes >= 4 * kMaxRow * 4, "row buffers fit the staging area");
  __shared__ __align__(16) char smem[kBytes];
  float4* spos = reinterpret_cast<float4*>(smem);
  uint64_t* skey = reinterpret_cast<uint64_t*>(smem + kCellCap * 16);
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int c = (int)xcd_block(blockIdx.x, gridDim.x);
  const int32_t a0 = cell_start[c], a1 = cell_start[c + 1];
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
  // stage candidate q of stencil cell v (vpre[v] <= q < vpre[v+1]); pad the keys to a power
  // of two for the sort. A thread's candidates (at most kCellCap / 256) first find their
  // stencil cells, then request their positions together.
  int p2 = 1;
  while (p2 < total) p2 <<= 1;
  constexpr int kPer = kCellCap / 256;
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
      // image-shifted position in fp32 (one rounding per axis)
      const float xs = p.x + (float)(code / 9 - 1) * (float)g.L[0];
      const float ys = p.y + (float)((code / 3) % 3 - 1) * (float)g.L[1];
      const float zs = p.z + (float)(code % 3 - 1) * (float)g.L[2];
      spos[q] = make_float4(xs, ys, zs, __uint_as_float(entry));
      if (FILL) skey[q] = ((uint64_t)entry << 32) | (uint32_t)q;
    } else if (FILL && q < p2) {
      skey[q] = ~0ull;
    }
  }
  __syncthreads();
  if (FILL) {  // bitonic sort of the keys (the entries of one stencil are distinct)
    for (int k = 2; k <= p2; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int u = t; u < (p2 >> 1); u += 256) {
          const int a = 2 * jj * (u / jj) + (u % jj);
          const int b = a + jj;
          const uint64_t va = skey[a], vb = skey[b];
          const bool up = (a & k) == 0;
          if ((va > vb) == up) { skey[a] = vb; skey[b] = va; }
        }
        __syncthreads();
      }
    }
  }
  // Each wave takes kCellAtoms of the cell's atoms at a time: every staged candidate read
  // from LDS is tested against all of them.
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int32_t k0 = a0 + wv * kCellAtoms; k0 < a1; k0 += 4 * kCellAtoms) {
    int32_t ia[kCellAtoms];
    float xf[kCellAtoms][3];
    int count[kCellAtoms];
    int64_t o[kCellAtoms];
#pragma unroll
    for (int u = 0; u < kCellAtoms; u++) {
      // atoms past the cell's end repeat its first atom (wave-uniform; never written)
      const int32_t i = cell_atoms[k0 + u < a1 ? k0 + u : a0];
      ia[u] = i;
      xf[u][0] = pos[3 * i];
      xf[u][1] = pos[3 * i + 1];
      xf[u][2] = pos[3 * i + 2];
      count[u] = 0;
      o[u] = FILL ? (int64_t)row_ptr[i] : 0;
    }
    for (int q0 = 0; q0 < total; q0 += 64) {
      const int q = q0 + lane;
      const bool ok = q < total;
      const int qs = ok ? (FILL ? (int)(uint32_t)skey[q] : q) : 0;
      const float4 p = spos[qs];
      const uint32_t entry = __float_as_uint(p.w);
      const int32_t j = (int32_t)(entry >> 5);
      const int code = (int)(entry & 31u);
#pragma unroll
      for (int u = 0; u < kCellAtoms; u++) {
        if (k0 + u >= a1) break;  // wave-uniform
        const float dx = p.x - xf[u][0], dy = p.y - xf[u][1], dz = p.z - xf[u][2];
        const float d2 = __builtin_fmaf(dz, dz, __builtin_fmaf(dy, dy, dx * dx));
        bool near = d2 < lo2;
        if (ok && !near && d2 <= hi2)  // inside the band: the fp64 test decides
          near = pair_pass(pos[3 * j], pos[3 * j + 1], pos[3 * j + 2], code, (double)xf[u][0],
                           (double)xf[u][1], (double)xf[u][2], g, rcs2);
        const bool pass = ok && near && !(j == ia[u] && code == 13);
        const uint64_t m = __ballot(pass);
        if (FILL && pass) {
          const int slot = count[u] + __popcll(m & lt);
          if (slot < kMaxRow) col_shift[o[u] + slot] = (uint32_t)j | ((uint32_t)code << 27);
        }
        count[u] += __popcll(m);
      }
    }
    if (!FILL && lane == 0) {
#pragma unroll
      for (int u = 0; u < kCellAtoms; u++)
        if (k0 + u < a1) row_ptr[ia[u]] = count[u];
    }
  }
}

// Longest row and total pair count of a scanned CSR: block reductions, one atomic of each
// per block. The scan adds in 32 bits, so a total beyond the int32 range of row_ptr wraps
// there; each row's count is still the difference of its (wrapped) bounds, and their 64-bit
// sum is the true total.
__global__ void __launch_bounds__(256) k_max_row(int32_t n, const int32_t* __restrict__ row_ptr,
                                                 int32_t* __restrict__ out,
                                                 unsigned long long* __restrict__ total) {
  int32_t i = blockIdx.x * 256 + threadIdx.x;
  int v = i < n ? (int)((uint32_t)row_ptr[i + 1] - (uint32_t)row_ptr[i]) : 0;
  unsigned long long s = (unsigned long long)v;
  for (int o = 32; o >= 1; o >>= 1) {
    v = max(v, __shfl_xor(v, o, 64));
    s += __shfl_xor(s, o, 64);
  }
  __shared__ int32_t sh[4];
  __shared__ unsigned long long ss[4];
  if ((threadIdx.x & 63) == 0) {
    sh[threadIdx.x >> 6] = v;
    ss[threadIdx.x >> 6] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicMax(out, max(max(sh[0], sh[1]), max(sh[2], sh[3])));
    atomicAdd(total, ss[0] + ss[1] + ss[2] + ss[3]);
  }
}

// rev[e] = slot of the reverse pair (j <- i, 26 - code) of entry e = (i <- j, code); rows are
// sorted by (j, code). Each pair is searched once, from the row of its smaller index: for an
// entry with j >= i the lane binary-searches row j for (i, 26 - code) and writes both
// directions. One wave takes kRevRows consecutive rows: their j >= i entries are compacted
// into LDS first, so every lane runs two interleaved searches (independent load chains).
constexpr int kRevRows = 2;
__global__ void __launch_bounds__(256) k_rev(int32_t n, const int32_t* __restrict__ row_ptr,
                                             const uint32_t* __restrict__ col,
                                             int32_t* __restrict__ rev) {
  __shared__ int32_t se[4][128];
  __shared__ uint32_t sw[4][128];
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
      if (ee < e_end) {
        int32_t r = i;
        while (row_ptr[r + 1] <= ee) r++;  // rows of the wave's range, ascending
        const uint32_t c = col[ee];
        const int32_t j = (int32_t)(c & 0x7FFFFFFu);
        want = j >= r;
        key = ((uint32_t)r << 5) | (26u - (c >> 27));
      }
      const uint64_t m = __ballot(want);
      if (want) {
        const int slot = cnt + __popcll(m & lt);
        se[wv][slot] = ee;
        sw[wv][slot] = key;
      }
      cnt += __popcll(m);
      e += 64;
    }
    base = e;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    int32_t lo[2], hi[2], ei[2];
    uint32_t want[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int k = lane + 64 * h;
      lo[h] = hi[h] = 0;
      ei[h] = -1;
      want[h] = 0;
      if (k < cnt) {
        ei[h] = se[wv][k];
        want[h] = sw[wv][k];
        const int32_t j = (int32_t)(col[ei[h]] & 0x7FFFFFFu);
        lo[h] = row_ptr[j];
        hi[h] = row_ptr[j + 1];
      }
    }
    while (lo[0] < hi[0] || lo[1] < hi[1]) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
        if (lo[h] < hi[h]) {
          const int32_t mid = (lo[h] + hi[h]) >> 1;
          const uint32_t cm = col[mid];
          const uint32_t km = ((cm & 0x7FFFFFFu) << 5) | (cm >> 27);
          if (km < want[h]) lo[h] = mid + 1; else hi[h] = mid;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
      if (ei[h] >= 0) {
        rev[ei[h]] = lo[h];
        rev[lo[h]] = ei[h];
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // the row of the next entries
    while (i < i1 - 1 && row_ptr[i + 1] <= base) i++;
  }
}

// ---- scan -----------------------------------------------------------------------------
constexpr int kScanTile = 4096;  // 256 threads x 16

__device__ __forceinline__ int32_t block_exclusive_scan_256(int32_t v, int32_t* sh, int32_t* total) {
  int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  int32_t off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    if (k < w) off += sh[k];
    tot += sh[k];
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// Two arrays of the same length can be scanned by the same launches: blockIdx.y (partial,
// final) or blockIdx.x (sums) selects the array, and its tile sums sit nb entries apart.
struct ScanPair {
  int32_t* d[2];
};

__global__ void __launch_bounds__(256) k_scan_partial(ScanPair sp, int64_t n,
                                                      int32_t* __restrict__ sums) {
  __shared__ int32_t sh[4];
  const int32_t* __restrict__ d = sp.d[blockIdx.y];
  int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * 16;
  int32_t s = 0;
  for (int k = 0; k < 16; k++)
    if (base + k < n) s += d[base + k];
  int32_t tot;
  block_exclusive_scan_256(s, sh, &tot);
  if (threadIdx.x == 0) sums[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = tot;
}

__global__ void __launch_bounds__(256) k_scan_sums(int32_t* __restrict__ sums_all, int32_t nb) {
  __shared__ int32_t sh[4];
  int32_t* __restrict__ sums = sums_all + (int64_t)blockIdx.x * nb;
  int32_t carry = 0;
  for (int32_t b0 = 0; b0 < nb; b0 += 256) {
    int32_t k = b0 + threadIdx.x;
    int32_t v = k < nb ? sums[k] : 0;
    int32_t tot;
    int32_t ex = block_exclusive_scan_256(v, sh, &tot);
    if (k < nb) sums[k] = carry + ex;
    carry += tot;
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) k_scan_final(ScanPair sp, int64_t n,
                                                    const int32_t* __restrict__ sums) {
  __shared__ int32_t sh[4];
  int32_t* __restrict__ d = sp.d[blockIdx.y];
  int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * 16;
  int32_t v[16];
  int32_t s = 0;
  for (int k = 0; k < 16; k++) {
    v[k] = (base + k < n) ? d[base + k] : 0;
    s += v[k];
  }
  int32_t tot;
  int32_t run = block_exclusive_scan_256(s, sh, &tot) +
                sums[(int64_t)blockIdx.y * gridDim.x + blockIdx.x];
  for (int k = 0; k < 16; k++) {
    if (base + k < n) d[base + k] = run;
    run += v[k];
  }
}

inline int32_t grid(int64_t n, int b) { return (int32_t)((n + b - 1) / b); }

}  // namespace

hipError_t scan_exclusive_i32(int32_t* data, int64_t n, int32_t* partial, hipStream_t s) {
  return scan_exclusive_i32_pair(data, nullptr, n, partial, s);
}

hipError_t scan_exclusive_i32_pair(int32_t* a, int32_t* b, int64_t n, int32_t* partial,
                                   hipStream_t s) {
  int32_t nb = grid(n, kScanTile);
  if (nb == 0) return hipSuccess;
  const unsigned na = b ? 2u : 1u;
  ScanPair sp{{a, b ? b : a}};
  k_scan_partial<<<dim3(nb, na), 256, 0, s>>>(sp, n, partial);
  k_scan_sums<<<na, 256, 0, s>>>(partial, nb);
  k_scan_final<<<dim3(nb, na), 256, 0, s>>>(sp, n, partial);
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
  // 1. wrap + keys
  k_wrap_key<<<grid(n, 256), 256, 0, st>>>(n, sort_curve(), L[0], L[1], L[2], pos, species,
                                           vel, forces,
                                           perm_accum, ws.pos_w, ws.key[0], ws.idx[0], ws.sp_tmp,
                                           ws.v_tmp, ws.f_tmp, ws.pa_tmp, status);
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
  // permute every per-atom array into sorted order
  k_permute<<<grid(n, 256), 256, 0, st>>>(n, ws.idx[cur], ws.key[cur], ws.pos_w, ws.sp_tmp,
                                          vel ? ws.v_tmp : nullptr, forces ? ws.f_tmp : nullptr,
                                          perm_accum ? ws.pa_tmp : nullptr, pos, species, vel,
                                          forces, perm_accum, ref_pos, perm, hkey);
  TESS_HIP_CHECK(hipGetLastError());
  // 3. cells
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
  TESS_HIP_CHECK(hipMemsetAsync(ws.cell_start, 0, sizeof(int32_t) * (ncell + 1), st));
  TESS_HIP_CHECK(hipMemsetAsync(ws.cell_fill, 0, sizeof(int32_t) * ncell, st));
  TESS_HIP_CHECK(hipMemsetAsync(ws.misc, 0, sizeof(int32_t) * 16, st));
  k_cell_count<<<grid(n, 256), 256, 0, st>>>(n, g, pos, ws.cell_id, ws.cell_start);
  TESS_HIP_CHECK(scan_exclusive_i32(ws.cell_start, ncell + 1, ws.scan_tmp, st));
  k_cell_fill<<<grid(n, 256), 256, 0, st>>>(n, ws.cell_id, ws.cell_start, ws.cell_fill,
                                            ws.cell_atoms, pos, ws.cell_pos);
  TESS_HIP_CHECK(hipGetLastError());
  // 4. pairs: count, scan, check, fill
  TESS_HIP_CHECK(hipMemsetAsync(row_ptr + n, 0, sizeof(int32_t), st));
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
  TESS_HIP_CHECK(scan_exclusive_i32(row_ptr, (int64_t)n + 1, ws.scan_tmp, st));
  // misc[0]: longest row; misc[4..5]: 64-bit pair total (the block is 256-byte aligned)
  unsigned long long* total = reinterpret_cast<unsigned long long*>(ws.misc + 4);
  k_max_row<<<grid(n, 256), 256, 0, st>>>(n, row_ptr, ws.misc, total);
  TESS_HIP_CHECK(hipGetLastError());
  int32_t max_row = 0, bits = 0;
  unsigned long long pairs = 0;
  TESS_HIP_CHECK(hipMemcpyAsync(&max_row, ws.misc, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  TESS_HIP_CHECK(hipMemcpyAsync(&pairs, total, sizeof(pairs), hipMemcpyDeviceToHost, st));
  TESS_HIP_CHECK(hipMemcpyAsync(&bits, status, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  TESS_HIP_CHECK(hipStreamSynchronize(st));
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
    k_rev<<<grid(n, 4 * kRevRows), 256, 0, st>>>(n, row_ptr, col_shift, rev);
    TESS_HIP_CHECK(hipGetLastError());
  }
  return TESS_OK;
}

}  // namespace tess
