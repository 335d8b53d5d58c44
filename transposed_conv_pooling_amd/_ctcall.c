/* _ctcall.c - CPython entry points that forward their arguments to the C ABI
 * of libct.so (include/ct.h), one function per compute entry point, with the
 * same argument order.  They only convert Python ints and floats to C types
 * and call the library: a per-call cost of well under a microsecond, where a
 * ctypes call with twenty-odd converted arguments costs a few.  Pointers and
 * the stream are passed as integers (0 for NULL); the return value is the
 * library's ct_status. */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

#include "ct.h"

#define P(v) ((void *)(uintptr_t)(v))

static PyObject *fused(PyObject *self, PyObject *args)
{
    unsigned long long x, w, cb, b, out, stream;
    int xdt, wdt, k, stride, pad, op, pk, ps;
    float s1, s2;
    long long N, Cin, D, H, W, Cout;
    (void)self;
    if (!PyArg_ParseTuple(args, "KiKiKKffLLLLLLiiiiiiKK", &x, &xdt, &w, &wdt, &cb, &b, &s1, &s2,
                          &N, &Cin, &D, &H, &W, &Cout, &k, &stride, &pad, &op, &pk, &ps, &out,
                          &stream))
        return NULL;
    return PyLong_FromLong(ct_convT3d_scale_pool_bias(P(x), xdt, P(w), wdt, (const float *)P(cb),
                                                      (const float *)P(b), s1, s2, N, Cin, D, H, W,
                                                      Cout, k, stride, pad, op, pk, ps,
                                                      (float *)P(out), P(stream)));
}

static PyObject *convT3d(PyObject *self, PyObject *args)
{
    unsigned long long x, w, b, out, stream;
    int xdt, wdt, k, stride, pad, op;
    long long N, Cin, D, H, W, Cout;
    (void)self;
    if (!PyArg_ParseTuple(args, "KiKiKLLLLLLiiiiKK", &x, &xdt, &w, &wdt, &b, &N, &Cin, &D, &H, &W,
                          &Cout, &k, &stride, &pad, &op, &out, &stream))
        return NULL;
    return PyLong_FromLong(ct_convT3d(P(x), xdt, P(w), wdt, (const float *)P(b), N, Cin, D, H, W,
                                      Cout, k, stride, pad, op, (float *)P(out), P(stream)));
}

static PyObject *avgpool3d(PyObject *self, PyObject *args)
{
    unsigned long long x, out, stream;
    int k, stride, pad, cip, bf16;
    long long N, C, D, H, W;
    (void)self;
    if (!PyArg_ParseTuple(args, "pKLLLLLiiiiKK", &bf16, &x, &N, &C, &D, &H, &W, &k, &stride, &pad,
                          &cip, &out, &stream))
        return NULL;
    if (bf16)
        return PyLong_FromLong(ct_avgpool3d_bf16((const uint16_t *)P(x), N, C, D, H, W, k, stride,
                                                 pad, cip, (uint16_t *)P(out), P(stream)));
    return PyLong_FromLong(ct_avgpool3d((const float *)P(x), N, C, D, H, W, k, stride, pad, cip,
                                        (float *)P(out), P(stream)));
}

static PyObject *convT1d(PyObject *self, PyObject *args)
{
    unsigned long long x, w, b, out, stream;
    int xdt, wdt, K, stride, pad, dil, op;
    long long N, Cin, L, Cout;
    (void)self;
    if (!PyArg_ParseTuple(args, "KiKiKLLLLiiiiiKK", &x, &xdt, &w, &wdt, &b, &N, &Cin, &L, &Cout,
                          &K, &stride, &pad, &dil, &op, &out, &stream))
        return NULL;
    return PyLong_FromLong(ct_convT1d(P(x), xdt, P(w), wdt, (const float *)P(b), N, Cin, L, Cout, K,
                                      stride, pad, dil, op, (float *)P(out), P(stream)));
}

static PyMethodDef methods[] = {
    {"fused", fused, METH_VARARGS, "ct_convT3d_scale_pool_bias"},
    {"convT3d", convT3d, METH_VARARGS, "ct_convT3d"},
    {"avgpool3d", avgpool3d, METH_VARARGS, "ct_avgpool3d / ct_avgpool3d_bf16"},
    {"convT1d", convT1d, METH_VARARGS, "ct_convT1d"},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_ctcall", NULL, -1, methods,
                                    NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__ctcall(void) { return PyModule_Create(&module); }
