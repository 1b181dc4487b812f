// rocrand_ref.cpp -- test-only host helper: Philox4x32-10 words and packed sign planes from
// rocRAND's open-source engine (rocrand/rocrand_philox4x32_10.h), an implementation
// independent of both the oracle and the library, used as a second check of the probe bits.
//
// The engine keyed with `seed`, at subsequence (probe | step << 32) and offset 4*blk, holds
// the Philox4x32-10 output for counter (blk_lo, blk_hi, probe, step) and key
// (seed_lo, seed_hi); its next four 32-bit draws are words 0..3 of that output.
#include <rocrand/rocrand_philox4x32_10.h>
#include <stdint.h>
#include <string.h>

extern "C" {

// out[4*i + w] = word w of the block blk0 + i, for i < nblk.
void rr_philox_words(uint64_t seed, uint32_t step, uint32_t probe, uint64_t blk0, uint64_t nblk,
                     uint32_t *out)
{
    for (uint64_t i = 0; i < nblk; ++i) {
        rocrand_device::philox4x32_10_engine eng(
            seed, (unsigned long long)probe | ((unsigned long long)step << 32),
            4ull * (blk0 + i));
        for (int w = 0; w < 4; ++w) out[4 * i + w] = eng();
    }
}

// The packed plane of one probe over params [offset, offset + n), offset a multiple of 128:
// ceil(n / 128) blocks of 16 bytes, each the four words stored little-endian.
void rr_plane(uint64_t seed, uint32_t step, uint32_t probe, uint64_t offset, uint64_t n,
              uint8_t *out)
{
    const uint64_t nblk = (n + 127) / 128;
    for (uint64_t i = 0; i < nblk; ++i) {
        uint32_t w[4];
        rr_philox_words(seed, step, probe, offset / 128 + i, 1, w);
        for (int k = 0; k < 4; ++k) {
            out[16 * i + 4 * k + 0] = (uint8_t)(w[k]);
            out[16 * i + 4 * k + 1] = (uint8_t)(w[k] >> 8);
            out[16 * i + 4 * k + 2] = (uint8_t)(w[k] >> 16);
            out[16 * i + 4 * k + 3] = (uint8_t)(w[k] >> 24);
        }
    }
}

}  // extern "C"
