/* Drives the oracle's C functions (oracle/oracle.c) with random small
 * inputs, valid and invalid (context lengths outside [1, 16 * max_blocks],
 * block ids outside the pool, copy pairs out of range), so that the build
 * under AddressSanitizer and UndefinedBehaviorSanitizer in
 * tests/test_host_sanitizers.py sees every access they make. Exits 0 when
 * every call returned; prints the number of calls and of error returns. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

uint64_t oracle_kv_bytes(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t);
int oracle_kv_append(uint16_t*, uint16_t*, const uint16_t*, const uint16_t*, const int32_t*,
                     const int32_t*, int, int, int, int, int);
int oracle_kv_write(uint16_t*, uint16_t*, const uint16_t*, const uint16_t*, const int32_t*,
                    const int32_t*, const int32_t*, int, int, int, int, int, int);
int oracle_copy_blocks(uint16_t*, uint16_t*, const int32_t*, const int32_t*, int, int, int, int);
int oracle_decode(double*, const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*,
                  const int32_t*, int, int, int, int, int, int, double);
int oracle_verify(double*, const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*,
                  const int32_t*, int, int, int, int, int, int, int, double);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {   /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static int pick(int lo, int hi) { return lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)); }
static uint16_t bf16_value(void) {  /* a finite bf16 of modest size */
  return (uint16_t)((next_u32() & 0x8000u) | (uint16_t)pick(0x3C00, 0x4080));
}

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? atoi(argv[1]) : 200;
  long calls = 0, errors = 0;
  for (int it = 0; it < rounds; ++it) {
    const int num_blocks = pick(4, 24), n_kv = pick(1, 3), group = pick(1, 4);
    const int n_q = n_kv * group, d = 8 * pick(1, 4), B = pick(1, 5), max_blocks = pick(1, 4);
    const size_t pool = (size_t)num_blocks * n_kv * 16 * d;
    uint16_t* k = malloc(pool * 2);
    uint16_t* v = malloc(pool * 2);
    for (size_t i = 0; i < pool; ++i) k[i] = bf16_value(), v[i] = bf16_value();
    int32_t* bt = malloc(sizeof(int32_t) * B * max_blocks);
    int32_t* cl = malloc(sizeof(int32_t) * B);
    const int bad_ids = pick(0, 3) == 0, bad_ctx = pick(0, 3) == 0;
    for (int i = 0; i < B * max_blocks; ++i)
      bt[i] = bad_ids ? pick(-2, num_blocks + 1) : pick(0, num_blocks - 1);
    for (int s = 0; s < B; ++s) cl[s] = bad_ctx ? pick(-1, 16 * max_blocks + 2) : pick(1, 16 * max_blocks);
    const int q_len = pick(1, 6);
    uint16_t* q = malloc(2 * (size_t)B * q_len * n_q * d);
    for (size_t i = 0; i < (size_t)B * q_len * n_q * d; ++i) q[i] = bf16_value();
    double* out = malloc(sizeof(double) * B * q_len * n_q * d);
    uint16_t* kn = malloc(2 * (size_t)B * n_kv * d);
    uint16_t* vn = malloc(2 * (size_t)B * n_kv * d);
    for (size_t i = 0; i < (size_t)B * n_kv * d; ++i) kn[i] = bf16_value(), vn[i] = bf16_value();

    errors += oracle_kv_append(k, v, kn, vn, bt, cl, B, max_blocks, num_blocks, n_kv, d) != 0;
    errors += oracle_decode(out, q, k, v, bt, cl, B, max_blocks, num_blocks, n_q, n_kv, d, 0.25) != 0;
    errors += oracle_verify(out, q, k, v, bt, cl, B, q_len, max_blocks, num_blocks, n_q, n_kv, d,
                            0.25) != 0;
    const int n_tok = pick(0, 6);
    int32_t rows[6], pos[6];
    for (int i = 0; i < n_tok; ++i) {
      rows[i] = pick(-1, B);
      pos[i] = pick(-1, 16 * max_blocks);
    }
    uint16_t* src = malloc(2 * (size_t)(n_tok + 1) * n_kv * d);
    for (size_t i = 0; i < (size_t)(n_tok + 1) * n_kv * d; ++i) src[i] = bf16_value();
    errors += oracle_kv_write(k, v, src, src, bt, rows, pos, n_tok, B, max_blocks, num_blocks, n_kv,
                              d) != 0;
    int32_t cs[4], cd[4];
    const int n_pairs = pick(0, 4);
    for (int i = 0; i < n_pairs; ++i) {
      cs[i] = pick(-1, num_blocks);
      cd[i] = pick(-1, num_blocks);
    }
    errors += oracle_copy_blocks(k, v, cs, cd, n_pairs, num_blocks, n_kv, d) != 0;
    (void)oracle_kv_bytes(pick(1, 80), n_kv, d, pick(1, 8192), B, 2);
    calls += 6;
    free(k); free(v); free(bt); free(cl); free(q); free(out); free(kn); free(vn); free(src);
  }
  printf("calls %ld errors %ld\n", calls, errors);
  return 0;
}
