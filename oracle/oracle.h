/*
 * oracle.h -- C interface of the fp64 CPU oracle (oracle.c).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, by __graft_entry__.smoke() and by
 * the cpu_baseline leg of bench.py, never by the product library.
 *
 * Layouts (all contiguous, row-major):
 *   q        [B][Sq][H][d]      k, v  [B][Skv][H][d]
 *   o        [B][n_rows][H][d]  lse   [B][H][n_rows]
 * where n_rows = Sq when rows == NULL, else the listed query rows in order.
 * All functions return 0 on success, -1 on a bad argument, -2 on allocation
 * failure.
 */
#ifndef ATTN_ORACLE_H
#define ATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_FP8_BLOCK 128

double oracle_bf16_to_double(uint16_t bits);
double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(double x);

int oracle_num_threads(void);
void oracle_set_num_threads(int n);

int oracle_attn_fwd_f64(const double* q, const double* k, const double* v,
                        double* o, double* lse,
                        int B, int H, int Sq, int Skv, int d, double scale,
                        const int* rows, int n_rows);

int oracle_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         double* o, double* lse,
                         int B, int H, int Sq, int Skv, int d, double scale,
                         const int* rows, int n_rows);

int oracle_attn_merge(const double* o_parts, const double* lse_parts, int n,
                      double* o, double* lse, int B, int H, int Sq, int d);

int oracle_quant_fp8(const uint16_t* x, uint8_t* q, float* scale,
                     int B, int H, int S, int d);

int oracle_dequant_fp8(const uint8_t* q, const float* scale, double* x,
                       int B, int H, int S, int d);

#ifdef __cplusplus
}
#endif

#endif
