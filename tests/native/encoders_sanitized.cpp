// Host-only check of the format encoders and the blob validator under
// AddressSanitizer / UndefinedBehaviorSanitizer (built by
// tests/test_native_sanitizers.py with g++; no GPU code is involved).
// Valid blobs of ragged shapes, all-kept / none-kept masks, -0 values and
// both tile widths are encoded, validated and turned into the column-run
// encoding; then truncated and bit-flipped copies of each blob go through the
// validator, and those it accepts through the column-run encoder.  The
// program exits non-zero if a valid blob is rejected; the sanitizers abort
// it on any invalid memory access or undefined behaviour.
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>
#include "swm_internal.h"
using namespace swm;
int main() {
  std::mt19937_64 rng(1234);
  int cases = 0, rejected = 0, accepted = 0;
  const int shapes[][2] = {{1, 1}, {16, 64}, {17, 65}, {300, 70}, {257, 1000}, {1100, 40}, {64, 4104}, {3, 2}, {1024, 2}};
  const double dens[] = {0.0, 0.3, 0.5, 1.0};
  for (auto& sh : shapes)
    for (double d : dens)
      for (int tkc = 0; tkc < 2; ++tkc) {
        const int64_t M = sh[0], K = sh[1];
        std::vector<uint16_t> W(M * K);
        std::vector<uint8_t> mask(M * K);
        std::uniform_real_distribution<double> u(0, 1);
        for (int64_t i = 0; i < M * K; ++i) {
          W[i] = uint16_t(rng() & 0xFFFF) & 0x7BFF;  // finite
          if (u(rng) < 0.05) W[i] = 0x8000;           // -0
          mask[i] = u(rng) < d;
        }
        swm_tile_cfg cfg{};
        cfg.tm = 16;
        cfg.tk = tkc ? 32 : 64;
        std::vector<uint8_t> blob;
        swm_status st = encode_blob(W.data(), K, mask.data(), K, M, K, &cfg, &blob);
        if (st != SWM_OK) { printf("encode status %d for %ldx%ld tk=%u\n", st, (long)M, (long)K, cfg.tk); continue; }
        Header h;
        if (validate_blob(blob.data(), blob.size(), &h) != SWM_OK) { printf("valid blob rejected\n"); return 1; }
        ColRunsHost c;
        st = colruns_from_tcb(blob.data(), blob.size(), &c);
        if (st == SWM_OK) {
          std::vector<uint8_t> out(colruns_blob_bytes(c));
          colruns_write_blob(c, out.data());
        }
        ++cases;
        // corrupted blobs: truncation and random byte flips
        for (int t = 0; t < 200; ++t) {
          std::vector<uint8_t> b = blob;
          if (t % 4 == 0) b.resize(rng() % (b.size() + 1));
          else for (int f = 0; f < 1 + int(rng() % 4); ++f) if (!b.empty()) b[rng() % b.size()] ^= uint8_t(1u << (rng() % 8));
          Header hh;
          if (validate_blob(b.data(), b.size(), &hh) == SWM_OK) {
            ++accepted;
            ColRunsHost cc;
            if (colruns_from_tcb(b.data(), b.size(), &cc) == SWM_OK) {
              std::vector<uint8_t> out(colruns_blob_bytes(cc));
              colruns_write_blob(cc, out.data());
            }
          } else ++rejected;
        }
      }
  printf("cases %d, corrupted accepted %d rejected %d\n", cases, accepted, rejected);
  return 0;
}
