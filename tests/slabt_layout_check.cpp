// Host-side check of the transposed slab operand's index arithmetic (the
// slabt_* functions of ttt_launch.h that the GEMM core's kSlabT loads and
// fragment reads use), with no GPU:
//  1. the per-lane / per-substep split of the transpose-read address equals
//     its definition;
//  2. emulating the direct-to-LDS loads (lane l of the load filling block b
//     writes the 16 bytes at LDS byte 1024 b + 16 l, copied from the HBM
//     piece slabt_piece_byte(b, lane) + slabt_step_byte(step) past the tile's
//     base) from an sb<256> matrix whose elements hold their own (row,
//     column), every element lands where slabt_lds_byte puts it, and every
//     piece stays inside the matrix;
//  3. emulating ds_read_b64_tr_b16 on that LDS image (lane i of a 16-lane
//     group receives, as its element e, element i % 4 of the 8 bytes that
//     lane 4e + i / 4 of the group addresses), each lane's 8-value B fragment
//     holds M[64 step + 8 kc + v][n0 + nb + lane % 32] for v = 0..7, kc =
//     2 sub + lane / 32;
//  4. no two lanes of one transpose read touch the same 16-byte bank group
//     of a 256-byte LDS line more than twice (the read moves 512 bytes, two
//     passes), and within each half-wave at most once per pass.
// Prints "ok" and exits 0, or prints the first mismatch and exits 1.
#include <cstdio>
#include <cstdint>
#include <vector>

#include "ttt_launch.h"

using namespace tttk;

static int fail(const char* what, long a, long b, long c, long d) {
  std::printf("FAIL %s: %ld %ld %ld %ld\n", what, a, b, c, d);
  return 1;
}

int main() {
  // 1. the split of the read address
  for (int lane = 0; lane < 64; ++lane)
    for (int nb = 0; nb < 256; nb += 32)
      for (int sub = 0; sub < 4; ++sub)
        for (int rd = 0; rd < 2; ++rd) {
          const uint32_t a = slabt_tr_byte(lane, nb, 2 * sub + lane / 32, rd);
          const uint32_t b = slabt_tr_lane(lane, nb, rd) + slabt_tr_sub(sub);
          if (a != b) return fail("tr split", lane, nb, sub, rd);
        }

  // An sb<256> matrix of R rows and K columns whose element (r, c) holds the
  // code r * K + c, read as a B tile at columns n0 .. n0 + 255.
  for (const int R : {256, 512, 320}) {
    for (const int K : {256, 512, 832}) {
      const int64_t elems = sb_elems<256>(R, K);
      std::vector<int64_t> M(elems, -1);
      for (int r = 0; r < R; ++r)
        for (int c = 0; c < K; ++c) M[sb_offset<256>(r, c, K)] = (int64_t)r * K + c;
      for (int n0 = 0; n0 < K; n0 += 256) {
        const int64_t base = (int64_t)(n0 / 64) * 256 * 64;  // tile base, elements
        for (int kl = 0; kl < R / 64; ++kl) {
          // 2. the loads
          std::vector<int64_t> lds(32 * 512, -2);
          for (int blk = 0; blk < 32; ++blk)
            for (int lane = 0; lane < 64; ++lane) {
              const int64_t src =
                  base + (slabt_piece_byte(blk, lane) + slabt_step_byte(kl, K)) / 2;
              const int64_t dst = blk * 512 + lane * 8;
              for (int e = 0; e < 8; ++e) {
                const int64_t s = src + e;
                // pieces past the matrix read as zero (buffer bound); only
                // columns past K may come from there
                const int64_t v = s < elems ? M[s] : -3;
                lds[dst + e] = v;
                // unwritten padding rows: only where columns past K alias
                if (v == -1 && n0 + 256 <= K) return fail("hole", blk, lane, kl, n0);
                if (v >= 0) {
                  const int r = (int)(v / K), c = (int)(v % K);
                  const int k = r - 64 * kl, n = c - n0;
                  // columns past K alias other rows; they feed only outputs
                  // that are never stored, and may sit anywhere
                  if (n0 + 256 <= K || c >= n0) {
                    if (k < 0 || k >= 64 || n < 0 || n >= 256)
                      return fail("piece outside the tile", blk, lane, r, c);
                    if (slabt_lds_byte(k, n) / 2 != dst + e)
                      return fail("lds position", k, n, blk, lane);
                  }
                } else if (v == -3 && n0 + 256 <= K) {
                  return fail("read past the matrix", blk, lane, kl, n0);
                }
              }
            }
          // 3. the fragments, and 4. the banks
          for (int nb = 0; nb < 256; nb += 32)
            for (int sub = 0; sub < 4; ++sub) {
              int64_t frag[64][8];
              for (int rd = 0; rd < 2; ++rd) {
                uint32_t addr[64];
                for (int lane = 0; lane < 64; ++lane) {
                  addr[lane] = slabt_tr_lane(lane, nb, rd) + slabt_tr_sub(sub);
                  if (addr[lane] % 8 != 0 || addr[lane] + 8 > 32768)
                    return fail("tr address", lane, nb, sub, rd);
                }
                int use[16] = {0};
                for (int half = 0; half < 2; ++half) {
                  int use_half[16] = {0};
                  for (int lane = 32 * half; lane < 32 * half + 32; ++lane) {
                    // a 16-byte group counts once per pair of lanes that read
                    // its two halves
                    if (addr[lane] % 16 != 0) continue;
                    const int slot = (addr[lane] / 16) % 16;
                    ++use[slot];
                    ++use_half[slot];
                  }
                  for (int s = 0; s < 16; ++s)
                    if (use_half[s] > 1) return fail("bank conflict in a half", nb, sub, rd, s);
                }
                for (int s = 0; s < 16; ++s)
                  if (use[s] > 2) return fail("bank conflict", nb, sub, rd, s);
                for (int lane = 0; lane < 64; ++lane) {
                  const int grp = lane / 16, i = lane % 16;
                  for (int e = 0; e < 4; ++e) {
                    const int src_lane = 16 * grp + 4 * e + i / 4;
                    frag[lane][4 * rd + e] = lds[addr[src_lane] / 2 + i % 4];
                  }
                }
              }
              for (int lane = 0; lane < 64; ++lane) {
                const int kc = 2 * sub + lane / 32, n = nb + lane % 32;
                if (n0 + n >= K) continue;
                for (int v = 0; v < 8; ++v) {
                  const int64_t want = (int64_t)(64 * kl + 8 * kc + v) * K + n0 + n;
                  if (frag[lane][v] != want) return fail("fragment", lane, nb, sub, v);
                }
              }
            }
        }
      }
    }
  }
  std::printf("ok\n");
  return 0;
}
